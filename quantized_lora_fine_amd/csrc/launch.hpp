// Kernel launchers of libnf4lora (implemented in the .hip files).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "nf4_host.hpp"

namespace nf4k {

enum { MODE_FWD = 0, MODE_DX = 1 };

hipError_t launch_quantize(const float* W, int64_t nblocks, bool dq, uint8_t* codes, void* absmax, float* dqs,
                           const NF4Consts& c, hipStream_t st);
hipError_t launch_dequantize(const uint8_t* codes, const void* absmax, const float* dqs, int64_t nweights, bool dq,
                             bool bf16, void* out, const NF4Consts& c, hipStream_t st);
hipError_t launch_error(const float* W, int64_t nblocks, bool dq, double* part, double* err, const NF4Consts& c,
                        hipStream_t st);
hipError_t launch_topk(const double* e, int n, int k, int* idx, hipStream_t st);

hipError_t launch_nf4_gemm(int mode, bool dq, const uint16_t* A, const uint8_t* codes, const void* absmax,
                           const float* dqs, const uint16_t* A2, const uint16_t* B2, int R, uint16_t* C, int64_t M,
                           int N, int K, const NF4Consts& c, hipStream_t st);

hipError_t launch_pad_transpose(const uint16_t* in, int64_t si, int64_t sj, int64_t irows, int64_t jcols,
                                uint16_t* out, int64_t orows, int64_t ocols, hipStream_t st);
void plan_nt(int64_t M, int K, int* ksplit, int* krange);
void plan_tn(int64_t M, int N, int* msplit, int64_t* mrange);
hipError_t launch_skinny_nt(const uint16_t* A, const uint16_t* B, int64_t M, int K, int RP, float* part, int ksplit,
                            int krange, hipStream_t st);
hipError_t launch_reduce_nt(const float* part, int64_t M, int RP, int r, int ksplit, float alpha1, uint16_t* out1,
                            int ld1, float alpha2, uint16_t* out2, hipStream_t st);
hipError_t launch_skinny_tn(const uint16_t* P, int ldp, int r, const uint16_t* Q, int64_t M, int N, int RP,
                            float* part, int msplit, int64_t mrange, hipStream_t st);
hipError_t launch_reduce_tn(const float* part, int RP, int r, int N, int msplit, float alpha, int trans, float* out,
                            hipStream_t st);

}  // namespace nf4k
