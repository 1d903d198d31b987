// C ABI of the library (declared in include/fa.h): argument validation,
// the gfx950 device check, and dispatch to the kernel launchers.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "fa_kernels.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = something else
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FA_ERR_DEVICE;
  }
  if (dev >= kMaxDevices) return FA_ERR_DEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FA_ERR_DEVICE;
    }
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? FA_OK : FA_ERR_DEVICE;
}

// Compute units of the current device (cached per device; 0 if unknown).
std::atomic<int> g_cus[kMaxDevices];
int device_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 0;
  }
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    g_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  const double elems = (double)B * (double)H * (double)N * (double)d;
  if (elems >= 1099511627776.0) return FA_ERR_SHAPE;  // 2^40
  // one (batch, head) slice is addressed with 32-bit byte offsets
  if ((double)N * (double)d * 2.0 >= 2147483648.0) return FA_ERR_SHAPE;
  // the grid is B * H * ceil(N / 128) workgroups
  if ((double)B * (double)H * (double)((N + 127) / 128) >= 2147483647.0) return FA_ERR_SHAPE;
  return FA_OK;
}

int check_scale(float s) { return (std::isfinite(s) && s > 0.f) ? FA_OK : FA_ERR_ARG; }

// sizes of the decode entry points (grouped KV heads, unequal lengths)
int check_decode_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  const bool dok = d == 64 || d == 128 || d == 256;
  const int dd = dok ? d : 1;
  if (Hkv < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (int e = check_shape(B, Hq, Nq, dd)) return e;
  if (int e = check_shape(B, Hkv, Nk, dd)) return e;
  if (Hq % Hkv) return FA_ERR_SHAPE;
  // 32-key tile offsets run up to 31 rows past the last key
  if ((double)(Nk + 32) * (double)dd * 2.0 >= 2147483648.0) return FA_ERR_SHAPE;
  if (!dok) return FA_ERR_HEADDIM;
  return FA_OK;
}

long long decode_workspace_bytes(int B, int Hq, int Nq, int d, int splits) {
  if (splits <= 1) return 0;
  return (long long)splits * B * Hq * Nq * (long long)(d + 1) * 4;
}

int launch_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  (void)hipGetLastError();
  return FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_PTR: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H and N must be >= 1 and the tensors smaller than 2^40 elements";
    case FA_ERR_HEADDIM: return "head dimension not supported by this entry point";
    case FA_ERR_ARG: return "invalid argument (causal must be 0/1, softmax_scale finite and > 0, known flags)";
    case FA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FA_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than the split count needs";
    case FA_ERR_SCRATCH: return "the split count needs more partial-result memory than the static 16 MiB scratch buffer holds";
    default: return "unknown status";
  }
}

int fa_fp8_vt_ld(int N) { return N < 1 ? 0 : ((N + 127) / 128) * 128; }

int fa_fp8_ref_block(int N, int causal) {
  if (N < 1) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  return fa::fwd_fp8_ref_block(N, causal == 1);
}

int fa_fwd_bf16(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int N, int d,
                int causal, float softmax_scale, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
  if (int e = check_shape(B, H, N, d == 64 || d == 128 || d == 256 ? d : 1)) return e;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int e = check_scale(softmax_scale)) return e;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  if (int e = check_device()) return e;

  fa::FwdBf16Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.N = N;
  p.Hkv = H;
  p.Nk = N;
  p.scale = softmax_scale;
  p.c = softmax_scale * 1.4426950408889634f;
  return launch_status(fa::launch_fwd_bf16(p, d, causal == 1, static_cast<hipStream_t>(stream)));
}

int fa_fwd_bf16_gqa(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq, int Hkv,
                    int Nq, int Nk, int d, int causal, float softmax_scale, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
  const int dd = d == 64 || d == 128 || d == 256 ? d : 1;
  if (Hkv < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (int e = check_shape(B, Hq, Nq, dd)) return e;
  if (int e = check_shape(B, Hkv, Nk, dd)) return e;
  if (Hq % Hkv) return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int e = check_scale(softmax_scale)) return e;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  if (int e = check_device()) return e;

  fa::FwdBf16Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = Hq;
  p.N = Nq;
  p.Hkv = Hkv;
  p.Nk = Nk;
  p.scale = softmax_scale;
  p.c = softmax_scale * 1.4426950408889634f;
  return launch_status(fa::launch_fwd_bf16(p, d, causal == 1, static_cast<hipStream_t>(stream)));
}

int fa_fwd_bf16_varlen(const void* q, const void* k, const void* v, float* o, float* lse, const int* cu_seqlens_q,
                       const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                       int d, int causal, float softmax_scale, void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL_PTR;
  const bool dok = d == 64 || d == 128 || d == 256;
  const double dd = dok ? d : 1;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || total_q < 0 || total_k < 0 || max_seqlen_q < 0) return FA_ERR_SHAPE;
  // Q and K/V rows of one sequence are addressed with 32-bit byte offsets
  // (a sequence's rows lie inside the packed tensors)
  if ((double)total_k * Hkv * dd * 2.0 >= 2147483648.0) return FA_ERR_SHAPE;
  if ((double)total_q * Hq * dd * 2.0 >= 2147483648.0) return FA_ERR_SHAPE;
  if ((double)total_q * Hq * dd >= 1099511627776.0) return FA_ERR_SHAPE;  // 2^40 elements
  if ((double)B * Hq * (((double)max_seqlen_q + 127) / 128) >= 2147483647.0) return FA_ERR_SHAPE;
  if (!dok) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int e = check_scale(softmax_scale)) return e;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) | reinterpret_cast<uintptr_t>(cu_seqlens_k)) & 3u) return FA_ERR_ALIGN;
  if (int e = check_device()) return e;

  fa::FwdBf16Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = Hq;
  p.N = max_seqlen_q;
  p.Hkv = Hkv;
  p.Nk = 0;
  p.scale = softmax_scale;
  p.c = softmax_scale * 1.4426950408889634f;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  return launch_status(fa::launch_fwd_bf16_varlen(p, d, causal == 1, static_cast<hipStream_t>(stream)));
}

int fa_fwd_bf16_decode_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits, int num_cus) {
  if (int e = check_decode_shape(B, Hq, Hkv, Nq, Nk, d)) return e;
  if (num_splits < 0 || num_cus < 0 || (num_splits == 0 && num_cus < 1)) return FA_ERR_ARG;
  return fa::dec_bf16_splits(B, Hq, Hkv, Nq, Nk, d, num_splits, num_cus);
}

long long fa_fwd_bf16_decode_workspace(int B, int Hq, int Nq, int d, int splits) {
  if (B < 1 || Hq < 1 || Nq < 1 || splits < 1 || (d != 64 && d != 128 && d != 256)) return FA_ERR_ARG;
  return decode_workspace_bytes(B, Hq, Nq, d, splits);
}

int fa_fwd_bf16_decode(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq, int Hkv,
                       int Nq, int Nk, int d, int causal, float softmax_scale, int num_splits, void* workspace,
                       long long workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
  if (int e = check_decode_shape(B, Hq, Hkv, Nq, Nk, d)) return e;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int e = check_scale(softmax_scale)) return e;
  if (num_splits < 1) return FA_ERR_ARG;
  const int splits = fa::dec_bf16_splits(B, Hq, Hkv, Nq, Nk, d, num_splits, 0);
  const double units = (double)B * Hkv * (((double)(Hq / Hkv) * Nq + 31) / 32);
  if (units * splits >= 2147483647.0) return FA_ERR_SHAPE;
  const long long need = decode_workspace_bytes(B, Hq, Nq, d, splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  if (need > 0 && !aligned16(workspace)) return FA_ERR_ALIGN;
  if (int e = check_device()) return e;

  fa::DecBf16Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = o;
  p.lse = lse;
  const size_t rows = (size_t)B * Hq * Nq;
  p.part_o = need > 0 ? static_cast<float*>(workspace) : nullptr;
  p.part_lse = need > 0 ? static_cast<float*>(workspace) + (size_t)splits * rows * d : nullptr;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.splits = splits;
  const int ntile = (Nk + 31) / 32;
  p.chunk_tiles = (ntile + splits - 1) / splits;
  p.scale = softmax_scale;
  p.c = softmax_scale * 1.4426950408889634f;
  return launch_status(fa::launch_dec_bf16(p, d, causal == 1, static_cast<hipStream_t>(stream)));
}

int fa_fwd_bf16_decode_noalloc(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq,
                               int Hkv, int Nq, int Nk, int d, int causal, float softmax_scale, int num_splits,
                               void* stream) {
  static_assert(FA_DECODE_SCRATCH_BYTES == fa::kDecScratchBytes, "header and library agree on the buffer size");
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
  if (int e = check_decode_shape(B, Hq, Hkv, Nq, Nk, d)) return e;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int e = check_scale(softmax_scale)) return e;
  if (num_splits < 0) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  if (int e = check_device()) return e;
  int splits;
  if (num_splits >= 1) {
    splits = fa::dec_bf16_splits(B, Hq, Hkv, Nq, Nk, d, num_splits, 0);
    if (decode_workspace_bytes(B, Hq, Nq, d, splits) > fa::kDecScratchBytes) return FA_ERR_SCRATCH;
  } else {
    const int cus = device_cus();
    if (cus < 1) return FA_ERR_DEVICE;
    splits = fa::dec_bf16_splits(B, Hq, Hkv, Nq, Nk, d, 0, cus);
    while (splits > 1 && decode_workspace_bytes(B, Hq, Nq, d, splits) > fa::kDecScratchBytes)
      splits = fa::dec_bf16_splits(B, Hq, Hkv, Nq, Nk, d, splits - 1, 0);
  }
  void* ws = nullptr;
  if (splits > 1) {
    if (fa::dec_scratch(&ws) != hipSuccess) {
      (void)hipGetLastError();
      return FA_ERR_DEVICE;
    }
  }
  // the workspace entry point with the same effective count: it checks the
  // rest and launches the same kernels
  return fa_fwd_bf16_decode(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, softmax_scale, splits, ws,
                            splits > 1 ? fa::kDecScratchBytes : 0, stream);
}

}  // extern "C"

namespace {

int bwd_common(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
               float* dq, float* dk, float* dv, float* delta_ws, int B, int H, int Hkv, int N, int d, int causal,
               float softmax_scale, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta_ws) return FA_ERR_NULL_PTR;
  if (int e = check_shape(B, H, N, d == 64 || d == 128 || d == 256 ? d : 1)) return e;
  if (Hkv < 1 || H % Hkv) return FA_ERR_SHAPE;
  // fp32 [N, d] slices are addressed with 32-bit byte offsets too
  if ((double)N * (double)d * 4.0 >= 2147483648.0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int e = check_scale(softmax_scale)) return e;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(delta_ws))
    return FA_ERR_ALIGN;
  if (int e = check_device()) return e;

  fa::BwdBf16Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.dout = static_cast<const uint16_t*>(dout);
  p.o = o;
  p.lse = lse;
  p.delta = delta_ws;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.B = B;
  p.H = H;
  p.N = N;
  p.Hkv = Hkv;
  p.scale = softmax_scale;
  p.c = softmax_scale * 1.4426950408889634f;
  // two dK/dV launches pay off once their grid (one workgroup per 128 keys
  // of a KV head) fills every CU; below that the single launch is faster
  const double wgs = (double)B * Hkv * ((N + 127) / 128);
  const int cus = device_cus();
  p.split_dkdv = (d == 128 && cus > 0 && wgs >= cus) ? 1 : 0;
  return launch_status(fa::launch_bwd_bf16(p, d, causal == 1, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int fa_bwd_bf16(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
                float* dq, float* dk, float* dv, float* delta_ws, int B, int H, int N, int d, int causal,
                float softmax_scale, void* stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, delta_ws, B, H, H, N, d, causal, softmax_scale, stream);
}

int fa_bwd_bf16_gqa(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
                    float* dq, float* dk, float* dv, float* delta_ws, int B, int Hq, int Hkv, int N, int d,
                    int causal, float softmax_scale, void* stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, causal, softmax_scale, stream);
}

int fa_fp8_prep(const void* x, void* x8, float* x_scale, const signed char* signs, int B, int H, int N, int d,
                unsigned flags, void* stream) {
  if (!x || !x8 || !x_scale) return FA_ERR_NULL_PTR;
  if (int e = check_shape(B, H, N, d == 128 ? d : 1)) return e;
  if (d != 128) return FA_ERR_HEADDIM;
  if (flags & ~(FA_PREP_TRANSPOSE | FA_PREP_PER_TENSOR | FA_PREP_POW2_SCALE)) return FA_ERR_ARG;
  if ((flags & FA_PREP_POW2_SCALE) && signs) return FA_ERR_ARG;
  if (!aligned16(x) || !aligned16(x8) || !aligned16(x_scale) || (signs && !aligned16(signs))) return FA_ERR_ALIGN;
  if (int e = check_device()) return e;

  fa::Fp8PrepParams p;
  p.x = static_cast<const uint16_t*>(x);
  p.x8 = static_cast<uint8_t*>(x8);
  p.scale = x_scale;
  p.signs = reinterpret_cast<const int8_t*>(signs);
  p.B = B;
  p.H = H;
  p.N = N;
  p.ld = fa_fp8_vt_ld(N);
  p.transpose = (flags & FA_PREP_TRANSPOSE) != 0;
  p.per_tensor = (flags & FA_PREP_PER_TENSOR) != 0;
  p.pow2 = (flags & FA_PREP_POW2_SCALE) != 0;
  return launch_status(fa::launch_fp8_prep(p, d, static_cast<hipStream_t>(stream)));
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* q_scale, const float* k_scale,
               const float* v_scale, float* o, float* lse, int B, int H, int N, int d, int causal,
               float softmax_scale, void* stream) {
  if (!q8 || !k8 || !v8t || !q_scale || !k_scale || !v_scale || !o || !lse) return FA_ERR_NULL_PTR;
  if (int e = check_shape(B, H, N, d == 128 ? d : 1)) return e;
  if (d != 128) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int e = check_scale(softmax_scale)) return e;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(q_scale) || !aligned16(k_scale) ||
      !aligned16(v_scale) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  if (int e = check_device()) return e;

  fa::FwdFp8Params p;
  p.q8 = static_cast<const uint8_t*>(q8);
  p.k8 = static_cast<const uint8_t*>(k8);
  p.v8t = static_cast<const uint8_t*>(v8t);
  p.qs = q_scale;
  p.ks = k_scale;
  p.vs = v_scale;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.N = N;
  p.ld = fa_fp8_vt_ld(N);
  p.scale = softmax_scale;
  p.c = softmax_scale * 1.4426950408889634f;
  return launch_status(fa::launch_fwd_fp8(p, d, causal == 1, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
