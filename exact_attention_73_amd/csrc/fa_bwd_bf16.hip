// Exact attention backward, bf16 operands, for gfx950 (MI355X).
//
// What is computed: the gradients of the forward O = softmax(scale Q K^T) V
// for an upstream gradient dO, using the row logsumexp the forward saved
// (so P is recomputed, never stored):
//   P = exp(scale Q K^T - lse),  D_i = sum_c dO_ic O_ic,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
// The pages list dQ, dK, dV among what a correct FA3 must cover
// ("FlashAttention-3：用异步流水榨出 Hopper 的 Attention 性能", section
// "正确性验证要覆盖异步边界") and report backward speed-ups (section
// "论文中的性能数字应该怎样理解"); the formulas are the derivative of the
// forward definition (wmrh.cn FlashAttention V3 article, section 一.1).
//
// Three kernels, no atomics:
//  * bwd_delta_kernel: D = rowsum(dO * O), one 16-lane group per row.
// Grouped heads (Hq = G Hkv query heads over Hkv KV heads, equal query and
// key lengths): a KV head's dK, dV are sums over the G query heads that read
// it, so a dK/dV workgroup streams the query tiles of all G heads through
// its ring into the same accumulators; dQ reads its query head's KV head.
//
//  * bwd_dkdv_kernel: one workgroup per (batch, KV head, 128 keys); each wave
//    owns 32 keys and keeps its K and V rows in VGPRs as B operands.  Query
//    tiles of 64 rows (Q, dO, lse, D) stream through a 2-slot LDS ring
//    filled by direct-to-LDS loads one tile ahead.  S = Q K^T and dP = dO V^T
//    are computed with the queries as rows, so a lane owns one key column and
//    P, dS leave the accumulators as the B operands of dV^T += dO^T P and
//    dK^T += Q^T dS, whose A operands come from transposed LDS reads of the
//    same tiles in the matching query order (the forward's PV trick).
//    At d = 128 a wave holding both accumulators needs more than 256
//    registers (one wave per SIMD).  When the grid has at least one
//    workgroup per CU the kernel runs as two launches instead, one
//    accumulating dV only (S and dV^T products) and one dK only (S, dP and
//    dK^T products, 32-query tiles): each fits 256 registers, so two waves
//    share every SIMD, which outweighs computing S twice.  The arithmetic
//    and its order are those of the single kernel, so results are the same
//    bit for bit.  At d = 256 the dK/dV work always runs as the two launches
//    (one wave per SIMD each; a single wave holding K, V and both 256-wide
//    accumulators would spill hundreds of registers).
//  * bwd_dq_kernel: shaped like the forward: one workgroup per 128 queries,
//    Q and dO resident as B operands, K and V tiles of 64 keys (32 at
//    d = 256) through the LDS ring; S^T = K Q^T, dP^T = V dO^T (a lane owns one query, so lse and
//    D are per-lane scalars) and dQ^T += K^T dS^T from transposed K reads.
// Causal: key tiles above a query tile (or query tiles before a key tile)
// are skipped; only tiles crossing the diagonal are masked element-wise.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_t;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16 bytes per lane from buffer offset voff straight into LDS at dst + 16 * lane
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)dst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* src) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t)src);
}

// XOR of the 16-byte chunk index of tile row r (rows of D bf16): the rows
// read by one ds_read_b128 spread over the LDS banks.
template <int D> __device__ __forceinline__ int swz(int r) {
  if constexpr (D == 64) return (r >> 1) & 7;
  else return r & 15;
}

// element offset of (row, col) in a swizzled [rows][D] bf16 tile
template <int D> __device__ __forceinline__ int tile_elem(int row, int col) {
  return row * D + (((col >> 3) ^ swz<D>(row)) << 3) + (col & 7);
}

// A operand of a 32x32x16 product whose k runs over tile rows: lane L gets
// column cbase + (L & 31) of rows {rbase + 4 hi + 0..3, rbase + 8 + 4 hi + 0..3}
// (hi = L >> 5), the key order in which P / dS leave the accumulators.
// Within a 16-lane group the transposed read hands lane i column cbase + i
// of the 4 rows that source lanes s = 4 e + i / 4 address.
template <int D> __device__ __forceinline__ bf16x8 read_cols(const uint16_t* t, int rbase, int cbase, int lane) {
  const int grp = lane >> 4, sl = lane & 15, hi = lane >> 5;
  const int col = cbase + 16 * (grp & 1) + 4 * (sl & 3);
  const int r0 = rbase + 4 * hi + (sl >> 2);
  const i16x4 a0 = lds_read_tr16(&t[tile_elem<D>(r0, col)]);
  const i16x4 a1 = lds_read_tr16(&t[tile_elem<D>(r0 + 8, col)]);
  const u32x2 w0 = __builtin_bit_cast(u32x2, a0), w1 = __builtin_bit_cast(u32x2, a1);
  return __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
}

// row operand (8 consecutive columns 16 s + 8 hi .. of tile row `row`)
template <int D> __device__ __forceinline__ bf16x8 read_row(const uint16_t* t, int row, int s, int hi) {
  return *reinterpret_cast<const bf16x8*>(&t[row * D + (((2 * s + hi) ^ swz<D>(row)) << 3)]);
}

// P, dS (fp32 accumulator registers 8 ks .. 8 ks + 7) as a bf16 B operand
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int ks) {
  u32x4 t;
#pragma unroll
  for (int h = 0; h < 4; ++h) t[h] = pack_bf16x2(x[8 * ks + 2 * h], x[8 * ks + 2 * h + 1]);
  return __builtin_bit_cast(bf16x8, t);
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ dout, const float* __restrict__ o,
                                                        float* __restrict__ delta, long rows) {
  constexpr int E = D / 16;  // elements per lane
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c0 = (threadIdx.x & 15) * E;
  float acc = 0.f;
  if (row < rows) {
    const uint16_t* g = dout + row * D + c0;
    const float* x = o + row * D + c0;
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(g + e);
      acc = __builtin_fmaf(__uint_as_float(w << 16), x[e], acc);
      acc = __builtin_fmaf(__uint_as_float(w & 0xffff0000u), x[e + 1], acc);
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && (threadIdx.x & 15) == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * 64;

// Workgroups per CU each kernel is compiled for (1: a wave may use up to 512
// registers and runs alone on its SIMD; 2: two waves share each SIMD and
// overlap each other's matrix and vector work).  At d = 128 the resident
// K, V rows and the dK, dV accumulators of a dK/dV wave need more than 256
// registers; the dQ kernel fits 256 at both head sizes (measured: two per
// CU is 18 % faster than one at d = 128).
// PART of the dK/dV work a launch does: both gradients, dV only, dK only.
enum DkdvPart { kBoth = 0, kDvOnly = 1, kDkOnly = 2 };

template <int D> struct BwdCfg {
  static constexpr int kDkdvMinb = D == 64 ? 2 : 1;  // both gradients in one wave
  // d = 256: Q and dO rows (128 registers) and the dQ accumulators (128)
  // leave a dQ wave more than 256 registers
  static constexpr int kDqMinb = D == 256 ? 1 : 2;
};
// the split launches fit two waves per SIMD at d = 128; at d = 256 a
// workgroup's 64 KB (dK) or 128 KB (dV) of tiles and its registers (K and V
// rows plus one accumulator: 256) allow one per CU
template <int D, int PART> constexpr int dkdv_minb() {
  return PART == kBoth ? BwdCfg<D>::kDkdvMinb : (D == 256 ? 1 : 2);
}
template <int PART> constexpr int dkdv_bq() { return PART == kDkOnly ? 32 : 64; }

template <int D, bool CAUSAL, int PART>
__global__ __launch_bounds__(kBwdThreads, (dkdv_minb<D, PART>())) void bwd_dkdv_kernel(BwdBf16Params p) {
  constexpr bool DO_V = PART != kDkOnly, DO_K = PART != kDvOnly;
  constexpr int BQ = dkdv_bq<PART>();  // queries per tile
  constexpr int NQB = BQ / 32;       // 32-query blocks per tile
  constexpr int NQS = D / 16;        // k-steps over d
  constexpr int NDB = D / 32;        // 32-row blocks of dK^T, dV^T
  constexpr int TILE = BQ * D;       // elements of a Q or dO tile
  constexpr int IPW = TILE * 2 / 1024 / kBwdWaves;  // 1 KB wave-loads per wave per tile
  constexpr int RPI = 1024 / (D * 2);               // rows per wave-load
  constexpr int CPR = D / 8;                        // 16-byte chunks per row

  __shared__ __attribute__((aligned(1024))) uint16_t Qs0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Qs1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Gs0[TILE];  // dO
  __shared__ __attribute__((aligned(1024))) uint16_t Gs1[TILE];
  __shared__ __attribute__((aligned(16))) float Ls0[BQ], Ls1[BQ], Ds0[BQ], Ds1[BQ];

  const int N = p.N;
  const int BK = p.B * p.Hkv;       // (batch, KV head) pairs
  const int G = p.H / p.Hkv;        // query heads per KV head
  const int nk = (N + 127) / 128;
  int bk, kt;
  if constexpr (CAUSAL) {
    // the first key tiles see the most query tiles: launch them first
    kt = (int)blockIdx.x / BK;
    bk = (int)blockIdx.x % BK;
  } else {
    const int w = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    bk = w / nk;
    kt = w % nk;
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const size_t base = (size_t)bk * N * D;  // k, v, dk, dv
  // query heads bk * G .. bk * G + G - 1 (b * Hq + h, adjacent) read this KV head
  const size_t qbh0 = (size_t)bk * G;
  const int kw0 = kt * 128 + wave * 32;  // first key of this wave
  const int key = kw0 + l32;             // the key column this lane owns

  // K and V rows of this lane's key as B operands (zero past N)
  bf16x8 kb[NQS], vb[NQS];
  {
    const bool ok = key < N;
    const u32x4* ks = reinterpret_cast<const u32x4*>(p.k + base + (size_t)(ok ? key : 0) * D);
    const u32x4* vs = reinterpret_cast<const u32x4*>(p.v + base + (size_t)(ok ? key : 0) * D);
#pragma unroll
    for (int s = 0; s < NQS; ++s) {
      kb[s] = __builtin_bit_cast(bf16x8, ok ? ks[2 * s + hi] : u32x4{0, 0, 0, 0});
      vb[s] = __builtin_bit_cast(bf16x8, ok ? vs[2 * s + hi] : u32x4{0, 0, 0, 0});
    }
  }

  const int nq = (N + BQ - 1) / BQ;
  const int j0 = CAUSAL ? (kt * 128) / BQ : 0;  // earlier query tiles see none of these keys
  const int nqh = nq - j0;                      // query tiles per query head
  const int ntl = G * nqh;                      // tiles streamed: every query head of the group

  // direct-to-LDS tile loads of tile t = (query head g, query tile j), each
  // through a buffer range of that head's N rows (rows past N read as zero)
  int off[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = (wave * IPW + i) * RPI + lane / CPR, pc = lane % CPR;
    off[i] = row * D * 2 + ((pc ^ swz<D>(row)) * 16);
  }
  auto issue = [&](uint16_t* qs, uint16_t* gs, float* ls, float* ds, int t) __attribute__((always_inline)) {
    const int g = t / nqh, j = j0 + t - g * nqh;
    const size_t hb = qbh0 + (size_t)g;
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(p.q + hb * N * D, N * D * 2);
    const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(p.dout + hb * N * D, N * D * 2);
    const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(p.lse + hb * N, N * 4);
    const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(p.delta + hb * N, N * 4);
    const int tb = j * BQ * D * 2;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      lds_dma16(rq, qs + (wave * IPW + i) * 512, off[i] + tb);
      lds_dma16(rg, gs + (wave * IPW + i) * 512, off[i] + tb);
    }
    // 64 floats of lse (wave 0) and D (wave 1): 16 lanes x 16 bytes
    if (wave == 0 && lane < BQ / 4) lds_dma16(rl, ls, (j * BQ + 4 * lane) * 4);
    if (wave == 1 && lane < BQ / 4) lds_dma16(rd, ds, (j * BQ + 4 * lane) * 4);
  };

  f32x16 dv[NDB], dk[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dv[db] = f32x16{};
    dk[db] = f32x16{};
  }
  const float c = p.c;

  auto step = [&](int t, const uint16_t* qs, const uint16_t* gs, const float* ls, const float* ds, uint16_t* qn,
                  uint16_t* gn, float* ln, float* dn) __attribute__((always_inline)) {
    wait_vmem_all();
    __syncthreads();  // tile t is in LDS; every wave is done with tile t - 1
    if (t + 1 < ntl) issue(qn, gn, ln, dn, t + 1);
    const int q0 = (j0 + t % nqh) * BQ;
    if (CAUSAL && q0 + BQ - 1 < kw0) return;  // every query of the tile precedes this wave's keys
    const bool need_mask = CAUSAL && q0 < kw0 + 31;

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const int row = qb * 32 + l32;
#pragma unroll
      for (int st = 0; st < NQS; ++st) {
        s = mfma_bf16_32x32x16(read_row<D>(qs, row, st, hi), kb[st], s);
        if constexpr (DO_K) dp = mfma_bf16_32x32x16(read_row<D>(gs, row, st, hi), vb[st], dp);
      }
      // register r holds query qb*32 + 8 (r / 4) + 4 hi + (r % 4)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&ls[qb * 32 + 8 * g + 4 * hi]);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(&ds[qb * 32 + 8 * g + 4 * hi]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = exp2_fast(__builtin_fmaf(s[r], c, -lv[e] * kLog2e));
          if (need_mask) {
            const int q = q0 + qb * 32 + 8 * g + 4 * hi + e;
            pv = key > q ? 0.f : pv;
          }
          s[r] = pv;
          if constexpr (DO_K) dp[r] = pv * (dp[r] - dd[e]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over this block's 32 queries
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int rbase = qb * 32 + 16 * ks;
        if constexpr (DO_V && DO_K) {
          const bf16x8 pb = pack8(s, ks), sb = pack8(dp, ks);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            dv[db] = mfma_bf16_32x32x16(read_cols<D>(gs, rbase, 32 * db, lane), pb, dv[db]);
            dk[db] = mfma_bf16_32x32x16(read_cols<D>(qs, rbase, 32 * db, lane), sb, dk[db]);
          }
        } else if constexpr (DO_V) {
          const bf16x8 pb = pack8(s, ks);
#pragma unroll
          for (int db = 0; db < NDB; ++db) dv[db] = mfma_bf16_32x32x16(read_cols<D>(gs, rbase, 32 * db, lane), pb, dv[db]);
        } else {
          const bf16x8 sb = pack8(dp, ks);
#pragma unroll
          for (int db = 0; db < NDB; ++db) dk[db] = mfma_bf16_32x32x16(read_cols<D>(qs, rbase, 32 * db, lane), sb, dk[db]);
        }
      }
    }
  };

  // Where a wave holds more than 256 registers its dK, dV accumulators live
  // in AGPRs; pinning them there at the loop's top and bottom (empty asm,
  // "a" constraint) stops the compiler from keeping vector-register copies
  // of them that it refreshes every iteration (about 300 AGPR moves per two
  // query tiles at d = 256 before, the 64 reads of S and dP after)
  auto pin = [&]() __attribute__((always_inline)) {
    if constexpr (D == 256 || (D == 128 && PART == kBoth)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if constexpr (DO_V) asm volatile("" : "+a"(dv[db]));
        if constexpr (DO_K) asm volatile("" : "+a"(dk[db]));
      }
    }
  };
  if (ntl > 0) {
    issue(Qs0, Gs0, Ls0, Ds0, 0);
    for (int t = 0; t < ntl; t += 2) {
      pin();
      step(t, Qs0, Gs0, Ls0, Ds0, Qs1, Gs1, Ls1, Ds1);
      if (t + 1 < ntl) step(t + 1, Qs1, Gs1, Ls1, Ds1, Qs0, Gs0, Ls0, Ds0);
      pin();
    }
  }

  // dK = scale dS^T Q, dV = P^T dO: lane holds key `key`, d = 32 db + 8 g + 4 hi + 0..3
  if (key < N) {
    float* dkr = p.dk + base + (size_t)key * D;
    float* dvr = p.dv + base + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 a = {dk[db][4 * g] * p.scale, dk[db][4 * g + 1] * p.scale, dk[db][4 * g + 2] * p.scale,
                         dk[db][4 * g + 3] * p.scale};
        const f32x4 b = {dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
        if constexpr (DO_K) *reinterpret_cast<f32x4*>(dkr + db * 32 + 8 * g + 4 * hi) = a;
        if constexpr (DO_V) *reinterpret_cast<f32x4*>(dvr + db * 32 + 8 * g + 4 * hi) = b;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, BwdCfg<D>::kDqMinb) void bwd_dq_kernel(BwdBf16Params p) {
  constexpr int BC = D == 256 ? 32 : 64;  // keys per tile (d = 256: two 16 KB tiles per slot)
  constexpr int NKB = BC / 32;
  constexpr int NQS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE = BC * D;
  constexpr int IPW = TILE * 2 / 1024 / kBwdWaves;
  constexpr int RPI = 1024 / (D * 2);
  constexpr int CPR = D / 8;

  __shared__ __attribute__((aligned(1024))) uint16_t Ks0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Ks1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs1[TILE];

  const int N = p.N;
  const int BH = p.B * p.H;
  const int nq = (N + 127) / 128;
  int bh, qt;
  if constexpr (CAUSAL) {
    qt = nq - 1 - (int)blockIdx.x / BH;  // heaviest query tiles first
    bh = (int)blockIdx.x % BH;
  } else {
    const int w = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    bh = w / nq;
    qt = w % nq;
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const size_t base = (size_t)bh * N * D;
  const int q0 = qt * 128 + wave * 32;
  const int qrow = q0 + l32;
  const bool qok = qrow < N;

  bf16x8 qb[NQS], gb[NQS];
  {
    const u32x4* qs = reinterpret_cast<const u32x4*>(p.q + base + (size_t)(qok ? qrow : 0) * D);
    const u32x4* gs = reinterpret_cast<const u32x4*>(p.dout + base + (size_t)(qok ? qrow : 0) * D);
#pragma unroll
    for (int s = 0; s < NQS; ++s) {
      qb[s] = __builtin_bit_cast(bf16x8, qok ? qs[2 * s + hi] : u32x4{0, 0, 0, 0});
      gb[s] = __builtin_bit_cast(bf16x8, qok ? gs[2 * s + hi] : u32x4{0, 0, 0, 0});
    }
  }
  const float lse2 = qok ? p.lse[(size_t)bh * N + qrow] * kLog2e : 0.f;
  const float dd = qok ? p.delta[(size_t)bh * N + qrow] : 0.f;

  const int kend = CAUSAL ? min(N, qt * 128 + 128) : N;
  const int ntiles = (kend + BC - 1) / BC;

  // KV head of this query head: each KV head serves H / Hkv consecutive query heads
  const int bb = bh / p.H, hh = bh - bb * p.H;
  const size_t kvbase = ((size_t)bb * p.Hkv + hh / (p.H / p.Hkv)) * N * D;
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.k + kvbase, N * D * 2);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(p.v + kvbase, N * D * 2);
  int off[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = (wave * IPW + i) * RPI + lane / CPR, pc = lane % CPR;
    off[i] = row * D * 2 + ((pc ^ swz<D>(row)) * 16);
  }
  auto issue = [&](uint16_t* ks, uint16_t* vs, int j) __attribute__((always_inline)) {
    const int tb = j * BC * D * 2;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      lds_dma16(rk, ks + (wave * IPW + i) * 512, off[i] + tb);
      lds_dma16(rv, vs + (wave * IPW + i) * 512, off[i] + tb);
    }
  };

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};
  const float c = p.c;

  auto step = [&](int j, const uint16_t* ks, const uint16_t* vs, uint16_t* kn, uint16_t* vn)
      __attribute__((always_inline)) {
    wait_vmem_all();
    __syncthreads();
    if (j + 1 < ntiles) issue(kn, vn, j + 1);
    const int key0 = j * BC;
    if (CAUSAL && key0 > q0 + 31) return;  // every key of the tile follows this wave's queries
    const bool need_mask = (CAUSAL && key0 + BC - 1 > q0) || (key0 + BC > N);

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const int row = kb * 32 + l32;
#pragma unroll
      for (int st = 0; st < NQS; ++st) {
        s = mfma_bf16_32x32x16(read_row<D>(ks, row, st, hi), qb[st], s);
        dp = mfma_bf16_32x32x16(read_row<D>(vs, row, st, hi), gb[st], dp);
      }
      // register r holds key key0 + kb*32 + 8 (r / 4) + 4 hi + (r % 4)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2_fast(__builtin_fmaf(s[r], c, -lse2));
        if (need_mask) {
          const int kk = key0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          pv = ((CAUSAL && kk > qrow) || kk >= N) ? 0.f : pv;
        }
        dp[r] = pv * (dp[r] - dd);
      }
      // dQ^T += K^T dS^T over this block's 32 keys
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 sb = pack8(dp, h);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dq[db] = mfma_bf16_32x32x16(read_cols<D>(ks, kb * 32 + 16 * h, 32 * db, lane), sb, dq[db]);
      }
    }
  };

  issue(Ks0, Vs0, 0);
  for (int j = 0; j < ntiles; j += 2) {
    // dQ accumulators in AGPRs at d = 256: pinned as in the dK/dV kernel
    if constexpr (D == 256) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) asm volatile("" : "+a"(dq[db]));
    }
    step(j, Ks0, Vs0, Ks1, Vs1);
    if (j + 1 < ntiles) step(j + 1, Ks1, Vs1, Ks0, Vs0);
    if constexpr (D == 256) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) asm volatile("" : "+a"(dq[db]));
    }
  }

  if (qok) {
    float* r = p.dq + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 a = {dq[db][4 * g] * p.scale, dq[db][4 * g + 1] * p.scale, dq[db][4 * g + 2] * p.scale,
                         dq[db][4 * g + 3] * p.scale};
        *reinterpret_cast<f32x4*>(r + db * 32 + 8 * g + 4 * hi) = a;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdBf16Params& p, hipStream_t stream) {
  const long rows = (long)p.B * p.H * p.N;
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, p.dout, p.o,
                     p.delta, rows);
  const unsigned bh = (unsigned)p.B * (unsigned)p.H;    // dQ: one workgroup per query head's 128 rows
  const unsigned bk = (unsigned)p.B * (unsigned)p.Hkv;  // dK/dV: one per KV head's 128 keys
  const unsigned tiles = (unsigned)((p.N + 127) / 128);
  // d = 256 always splits: one wave holding K, V and both accumulators
  // (512 registers of state) spills hundreds of registers
  if constexpr (D == 256) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, kDvOnly>), dim3(bk * tiles), dim3(kBwdThreads), 0, stream, p);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, kDkOnly>), dim3(bk * tiles), dim3(kBwdThreads), 0, stream, p);
  } else {
    bool split = false;
    if constexpr (D == 128) {
      if (p.split_dkdv) {
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, kDvOnly>), dim3(bk * tiles), dim3(kBwdThreads), 0, stream, p);
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, kDkOnly>), dim3(bk * tiles), dim3(kBwdThreads), 0, stream, p);
        split = true;
      }
    }
    if (!split) hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, kBoth>), dim3(bk * tiles), dim3(kBwdThreads), 0, stream, p);
  }
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(bh * tiles), dim3(kBwdThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdBf16Params& p, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 64: return causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
    case 128: return causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
    case 256: return causal ? launch<256, true>(p, stream) : launch<256, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
