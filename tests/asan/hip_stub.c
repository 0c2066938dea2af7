/*
 * Stand-in for the HIP runtime under the sanitizer build of the library's
 * host code (compiled host-only, so it carries no device code object).
 *
 * The module constructors that every HIP translation unit emits register
 * their (absent) code object, kernels and device variables at load time:
 * those calls do nothing here.  Any other HIP runtime entry point the host
 * code references gets a generated trap (see test_host_sanitizers.py) that
 * reports its name and aborts, so a validation path that reached the
 * runtime fails loudly instead of passing.
 */
#include <stddef.h>

void** __hipRegisterFatBinary(const void* wrapper) {
  (void)wrapper;
  static void* handle = NULL;
  return &handle;
}

void __hipUnregisterFatBinary(void** handle) { (void)handle; }

void __hipRegisterFunction(void** handle, const void* host_fn, char* device_fn,
                           const char* device_name, unsigned int thread_limit, void* tid,
                           void* bid, void* block_dim, void* grid_dim, int* wsize) {
  (void)handle; (void)host_fn; (void)device_fn; (void)device_name; (void)thread_limit;
  (void)tid; (void)bid; (void)block_dim; (void)grid_dim; (void)wsize;
}

void __hipRegisterVar(void** handle, char* host_var, char* device_address,
                      const char* device_name, int ext, size_t size, int constant, int global) {
  (void)handle; (void)host_var; (void)device_address; (void)device_name; (void)ext;
  (void)size; (void)constant; (void)global;
}
