// Host-side launch entry points of the gfx950 kernels (internal to the
// library; the public C ABI is include/fa.h).  Arguments have been validated
// by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdBf16Params {
  const uint16_t* q;  // bf16 [B, H, N, d]
  const uint16_t* k;  // bf16 [B, Hkv, Nk, d]
  const uint16_t* v;
  float* o;    // fp32 [B, H, N, d]
  float* lse;  // fp32 [B, H, N]
  int B, H, N;
  int Hkv, Nk;   // KV heads (H a multiple of Hkv) and keys; query i sees keys j <= i + Nk - N when causal
  float scale;   // softmax scale
  float c;       // scale * log2(e)
  // packed variable-length batch (launch_fwd_bf16_varlen): q, o [total_q, H, d],
  // k, v [total_k, Hkv, d], lse [H, total_q]; sequence b owns rows cu_q[b] ..
  // cu_q[b+1] - 1 and cu_k[b] .. cu_k[b+1] - 1; B sequences, N = longest query count
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int total_q = 0, total_k = 0;
};

hipError_t launch_fwd_bf16(const FwdBf16Params& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_bf16_varlen(const FwdBf16Params& p, int d, bool causal, hipStream_t stream);

struct DecBf16Params {
  const uint16_t* q;  // bf16 [B, Hq, Nq, d]
  const uint16_t* k;  // bf16 [B, Hkv, Nk, d]
  const uint16_t* v;
  float* o;           // fp32 [B, Hq, Nq, d]
  float* lse;         // fp32 [B, Hq, Nq]
  float* part_o;      // fp32 [splits, B * Hq * Nq, d] chunk results (splits > 1)
  float* part_lse;    // fp32 [splits, B * Hq * Nq]
  int B, Hq, Hkv, Nq, Nk;
  int splits;       // key chunks per KV head (non-empty)
  int chunk_tiles;  // 32-key tiles per chunk
  float scale;      // softmax scale
  float c;          // scale * log2(e)
};

hipError_t launch_dec_bf16(const DecBf16Params& p, int d, bool causal, hipStream_t stream);
// Bytes of the library's static per-device scratch buffer for decode
// partials, and its device address on the current device (looked up once
// per device).
constexpr long long kDecScratchBytes = 16ll << 20;
hipError_t dec_scratch(void** ptr);
// Key chunks per KV head: `requested` >= 1 reduced to the non-empty count,
// or 0 for the cost model's choice on a device with num_cus compute units.
int dec_bf16_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int requested, int num_cus);

struct BwdBf16Params {
  const uint16_t* q;     // bf16 [B, H, N, d]
  const uint16_t* k;     // bf16 [B, Hkv, N, d]
  const uint16_t* v;
  const uint16_t* dout;  // bf16 [B, H, N, d], upstream gradient
  const float* o;        // fp32 [B, H, N, d], forward output
  const float* lse;      // fp32 [B, H, N], forward logsumexp (natural log)
  float* delta;          // fp32 [B, H, N] workspace: rowsum(dO * O)
  float* dq;             // fp32 [B, H, N, d]
  float* dk;             // fp32 [B, Hkv, N, d]
  float* dv;
  int B, H, N;
  int Hkv;               // KV heads (H a multiple of Hkv); k, v are [B, Hkv, N, d]
  float scale;  // softmax scale
  float c;      // scale * log2(e)
  int split_dkdv;  // d = 128: dV and dK in two launches (set when the grid fills the device)
};

hipError_t launch_bwd_bf16(const BwdBf16Params& p, int d, bool causal, hipStream_t stream);

struct Fp8PrepParams {
  const uint16_t* x;   // bf16 [B, H, N, d]
  uint8_t* x8;         // E4M3 codes, [B, H, N, d] or [B, H, d, ld]
  float* scale;        // fp32 [B, H, nb]
  const int8_t* signs; // [H, d] or nullptr
  int B, H, N, ld;
  bool transpose;
  bool per_tensor;
  bool pow2;  // power-of-two scales (no rotation)
};

hipError_t launch_fp8_prep(const Fp8PrepParams& p, int d, hipStream_t stream);

struct FwdFp8Params {
  const uint8_t* q8;  // [B, H, N, d]
  const uint8_t* k8;  // [B, H, N, d]
  const uint8_t* v8t; // [B, H, d, ld]
  const float* qs;    // [B, H, nb]
  const float* ks;
  const float* vs;
  float* o;
  float* lse;
  int B, H, N, ld;
  float scale;
  float c;
};

hipError_t launch_fwd_fp8(const FwdFp8Params& p, int d, bool causal, hipStream_t stream);
// which forward kernel launch_fwd_fp8 runs, and the keys per exponent-reference
// step it implies (the tile of that kernel)
bool fwd_fp8_pingpong(int N, bool causal);
int fwd_fp8_ref_block(int N, bool causal);

}  // namespace fa
