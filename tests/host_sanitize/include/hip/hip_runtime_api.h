/* Test-only stand-in for the HIP runtime header: the few types and calls the
 * C-ABI layer (fa_api.cpp) uses, so that it can be compiled by the host
 * compiler alone under AddressSanitizer / UndefinedBehaviorSanitizer /
 * ThreadSanitizer and linked against sim_device.cpp, a simulated device
 * whose "device memory" is host memory.  Never used by the library build. */
#ifndef FA_TEST_SIM_HIP_RUNTIME_API_H_
#define FA_TEST_SIM_HIP_RUNTIME_API_H_

#include <stddef.h>

typedef enum hipError_t {
    hipSuccess = 0,
    hipErrorInvalidValue = 1,
    hipErrorOutOfMemory = 2,
    hipErrorNoDevice = 100,
    hipErrorInvalidDevice = 101,
    hipErrorInvalidSymbol = 701
} hipError_t;

typedef struct ihipStream_t *hipStream_t;

typedef struct hipDeviceProp_t {
    char name[256];
    char gcnArchName[256];
    int multiProcessorCount;
} hipDeviceProp_t;

#ifdef __cplusplus
extern "C" {
#endif
hipError_t hipGetDevice(int *device);
hipError_t hipSetDevice(int device);
hipError_t hipGetDeviceProperties(hipDeviceProp_t *prop, int device);
const char *hipGetErrorString(hipError_t e);
hipError_t hipMalloc(void **ptr, size_t size);
hipError_t hipFree(void *ptr);
#ifdef __cplusplus
}
#endif

#endif
