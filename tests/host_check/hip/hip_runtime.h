/*
 * Host-only stand-in for the few HIP runtime names that qmat_api.cpp and
 * qmat_launch.hpp use, so that the C ABI's argument checks can be compiled
 * by g++ with AddressSanitizer and UndefinedBehaviorSanitizer and run on a
 * machine without a GPU (tests/test_sanitizers.py). It declares no kernels
 * and runs nothing on a device; the launchers are stubs that count calls
 * (launch_stub.cpp).
 */
#ifndef QMAT_HOST_CHECK_HIP_RUNTIME_H
#define QMAT_HOST_CHECK_HIP_RUNTIME_H

#include <stdint.h>

typedef enum hipError_t { hipSuccess = 0, hipErrorUnknown = 999 } hipError_t;
typedef struct ihipStream_t* hipStream_t;

#define __device__
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) ((const void*)&(x))

hipError_t hipGetDevice(int* dev);
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol);

#endif
