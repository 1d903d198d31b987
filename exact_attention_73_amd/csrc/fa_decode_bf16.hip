// Decode-shaped attention forward (bf16 operands, fp32 O and lse) for
// gfx950: a few queries per head against a long key/value sequence, with
// grouped- or multi-query KV heads.
//
// What is computed is exactly the forward of fa_fwd_bf16_gqa: for query
// head h (KV head h / (Hq / Hkv)) and query i, O = softmax(scale q_i K^T) V
// over the keys j <= i + Nk - Nq (causal, bottom-right) or all keys, and
// lse = ln sum_j exp(scale q_i . k_j).  Only the work decomposition differs.
// The FA3 explainer (sections "GQA/MQA 为何改变 Kernel 任务数量" and
// "Prefill、Decode 和训练的收益不同") notes that a one-token query against a
// long KV cache is dominated by reading K and V, that a grid over batch x
// head x query tile then has too few tasks, and that query-head packing and
// split-KV are what give such shapes enough parallelism.  This kernel does
// both:
//
//  * Query-head packing: the G = Hq / Hkv query heads that read one KV head
//    are adjacent in [B, Hq, Nq, d], so their G * Nq query rows form one
//    contiguous list of R rows.  Blocks of 32 of them are the column
//    dimension of one matrix product, and each K/V tile read from HBM
//    serves up to 32 rows at once.
//  * Split-KV: the 32-key tiles of one KV head are cut into `splits` chunks
//    of chunk_tiles tiles.  There is one workgroup per (batch, KV head,
//    chunk, 32-row block), and the waves of a workgroup take interleaved
//    tiles of the chunk (wave w: tiles w, w + NW, ...).  Each wave streams
//    its tiles through a private 2-slot LDS ring with direct-to-LDS buffer
//    loads, so no barrier sits in the loop, and it keeps its own running
//    max, sum and accumulator.
//  * Merges: at the end the NW waves are merged through LDS.  A workgroup
//    then writes either the final O and lse (one chunk) or its chunk's
//    normalised O_c and lse_c.  A second kernel combines chunks with
//    lse = ln sum_c exp(lse_c) and O = sum_c exp(lse_c - lse) O_c.  This is
//    the online-softmax merge rule (FA3 explainer, section "Online Softmax
//    仍是精确合并的核心"), applied to whole chunks.
//
// Per wave the products are the transposed ones of the prefill kernel:
// S^T = K Q^T (lane L owns packed row L & 31 and 16 of the 32 keys of the
// tile) and O^T = V^T P^T with V read through ds_read_b64_tr_b16.  The key
// order of the P^T registers matches the order of those reads.  With at
// most 32 useful rows per product, the matrix cores idle most of the time;
// the kernel is bound by HBM reads of K and V.
#include <atomic>
#include <cmath>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kTileKeys = 32;  // keys per tile (one 32-key block of S^T)

// NW waves per workgroup and MINB workgroups per CU.  Two ring slots of
// K and V per wave: 2 * NW * 2 * 32 * d * 2 bytes of LDS = 128 KB (d = 128,
// 256) or 64 KB (d = 64), which bounds how many tiles are in flight per CU.
template <int D> struct DecCfg;
template <> struct DecCfg<64> {
  static constexpr int NW = 4, MINB = 2;
};
template <> struct DecCfg<128> {
  static constexpr int NW = 4, MINB = 1;
};
template <> struct DecCfg<256> {
  static constexpr int NW = 2, MINB = 1;
};

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_t;

// XOR of the 16-byte chunk index of K row r (conflict-free ds_read_b128 of
// the A operand) and of V row r (matched to the transposed read).
template <int D> __device__ __forceinline__ int k_swizzle(int r) {
  if constexpr (D == 64) return (r >> 1) & 7;
  else return r & 15;
}
template <int D> __device__ __forceinline__ int v_swizzle(int r) {
  if constexpr (D == 64) return ((r >> 1) & 1) << 2;
  else return (r & 3) << 2;
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left alone), through the builtin so
// that the compiler's own counter bookkeeping sees it
template <int N> __device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// 16 bytes per lane from buffer offset voff straight into LDS at dst + 16 * lane,
// with the non-temporal cache policy (cache-policy bit 1): K and V are read
// exactly once per call, so they stream past the caches.  Measured on
// MI355X: 12-14 % faster than the default policy on K/V sets larger than
// the last-level cache.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint16_t* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)dst, 16, voff, 0, 0, 2);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* src) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t)src);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(DecCfg<D>::NW * 64, DecCfg<D>::MINB) void dec_bf16_kernel(DecBf16Params p) {
  constexpr int NW = DecCfg<D>::NW;
  constexpr int TK = kTileKeys;
  constexpr int ROWB = D * 2;              // bytes per K/V row
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;         // rows per 1 KB wave-load
  constexpr int LPT = TK * ROWB / 1024;    // wave-loads per K (or V) tile
  constexpr int NDB = D / 32;              // 32-row blocks of O^T
  constexpr int NQS = D / 16;              // k-steps of S^T = K Q^T
  constexpr int TILE = TK * D;             // elements of one K or V tile
  static_assert(2 * LPT < 64, "the wait counts of one tile fit vmcnt");
  // slot s: K of wave w at [w * TILE], V of wave w at [(NW + w) * TILE]
  __shared__ __attribute__((aligned(1024))) uint16_t S0[2 * NW * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t S1[2 * NW * TILE];
  static_assert((NW * 64 + (NW - 1) * NDB * 16 * 64) * 4 <= 2 * NW * TILE * 2, "the merge fits in slot 0");

  const int G = p.Hq / p.Hkv;
  const int Nq = p.Nq, Nk = p.Nk;
  const int R = G * Nq;                 // packed rows per KV head
  const int nrb = (R + 31) / 32;        // 32-row blocks
  // work item: row block fastest, then chunk, then (batch, KV head); the
  // XCD-contiguous order keeps the row blocks of one chunk on one L2
  const int w_id = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
  const int rb = w_id % nrb;
  const int rest = w_id / nrb;
  const int split = rest % p.splits;
  const int bk = rest / p.splits;  // b * Hkv + KV head
  const int b = bk / p.Hkv, hkv = bk - b * p.Hkv;

  const int tid = threadIdx.x;
  // the wave index is uniform across the wave: keep it (and the tile counts
  // derived from it) in scalar registers so the loop branches are scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int off = Nk - Nq;  // causal: query i sees keys j <= i + off
  const size_t row0 = ((size_t)b * p.Hq + (size_t)hkv * G) * Nq;  // first packed row in [B * Hq * Nq]
  const int r = rb * 32 + l32;  // this lane's packed row
  const bool rok = r < R;
  const int qi = r % Nq;  // its query index

  // Q^T as B operands for the whole loop: k-step s holds d = 16 s + 8 hi .. +7
  bf16x8 qreg[NQS];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(p.q + (row0 + (size_t)(rok ? r : 0)) * D);
#pragma unroll
    for (int s = 0; s < NQS; ++s) {
      const u32x4 t = rok ? src[2 * s + hi] : u32x4{0, 0, 0, 0};
      qreg[s] = __builtin_bit_cast(bf16x8, t);
    }
  }

  // this chunk's tiles, and this wave's share of them
  const int ntile = (Nk + TK - 1) / TK;
  const int t_beg = split * p.chunk_tiles;
  const int t_end = min(ntile, t_beg + p.chunk_tiles);
  const int n_my = t_end - t_beg > wave ? (t_end - t_beg - wave + NW - 1) / NW : 0;
  auto tile_of = [&](int i) { return t_beg + wave + NW * i; };

  // direct-to-LDS loads: wave-load i fills 1 KB of the wave's tile, RPI rows;
  // lane L writes physical chunk L % CPR of row i * RPI + L / CPR and fetches
  // the logical chunk the swizzle puts there.  Rows past Nk read as zero.
  const size_t kvbase = (size_t)bk * Nk * D;
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.k + kvbase, Nk * ROWB);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(p.v + kvbase, Nk * ROWB);
  int koff[LPT], voff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int row = i * RPI + lane / CPR, pc = lane % CPR;
    koff[i] = row * ROWB + ((pc ^ k_swizzle<D>(row)) * 16);
    voff[i] = row * ROWB + ((pc ^ v_swizzle<D>(row)) * 16);
  }
  // This wave's i-th tile into slot.  Past its last tile the loads still
  // issue, at the end of the buffer's range, where they read zeros without
  // touching memory: every step then has the same number of loads in
  // flight behind it and waits with one fixed count.
  auto issue = [&](uint16_t* slot, int i) {
    const int base = i < n_my ? tile_of(i) * TK * ROWB : Nk * ROWB;
#pragma unroll
    for (int j = 0; j < LPT; ++j) lds_dma16(rk, slot + wave * TILE + j * 512, koff[j] + base);
#pragma unroll
    for (int j = 0; j < LPT; ++j) lds_dma16(rv, slot + (NW + wave) * TILE + j * 512, voff[j] + base);
  };

  // V^T A operand via the transposed read: within each 16-lane group, source
  // lane s addresses row kbase + s/4, columns dbase + 4 (s%4) .. +3; lane i of
  // the group then receives column dbase + i, rows kbase .. kbase + 3.
  const int grp = lane >> 4, sl = lane & 15;
  const int v_row_in = sl >> 2;
  const int v_col_in = 16 * (grp & 1) + 4 * (sl & 3);
  auto read_vt = [&](const uint16_t* vs, int kbase, int db) __attribute__((always_inline)) -> i16x4 {
    const int row = kbase + v_row_in;
    const int col = 32 * db + v_col_in;
    const int e = row * D + (((col >> 3) ^ v_swizzle<D>(row)) << 3) + (col & 7);
    return lds_read_tr16(&vs[e]);
  };

  float m_run = -INFINITY;  // running max (raw score units) of this wave's keys
  float l_run = 0.f;        // this half-wave's share of the running sum
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  const float c = p.c;
  const float lazy = kLazyLog2 / c;  // the rescale threshold in raw score units

  auto step = [&](int i, uint16_t* slot) {
    wait_vmem<2 * LPT>();  // tile i has landed; only tile i + 1's loads may be outstanding
    const uint16_t* ks = slot + wave * TILE;
    const uint16_t* vs = slot + (NW + wave) * TILE;
    const int key0 = tile_of(i) * TK;

    f32x16 s = {};
#pragma unroll
    for (int st = 0; st < NQS; ++st) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&ks[l32 * D + (((2 * st + hi) ^ k_swizzle<D>(l32)) * 8)]);
      s = mfma_bf16_32x32x16(a, qreg[st], s);
    }
    // keys past Nk, and (causal) keys after the query's last visible key
    if ((CAUSAL && key0 + TK - 1 > off) || key0 + TK > Nk) {
      // key = key0 + 4 hi + k, k a constant per register: dead iff k > lim
      int lim = Nk - 1 - key0 - 4 * hi;
      if constexpr (CAUSAL) lim = min(lim, qi + off - key0 - 4 * hi);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int k = 8 * (rr >> 2) + (rr & 3);
        s[rr] = k > lim ? -INFINITY : s[rr];
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int rr = 0; rr < 16; rr += 2) mx = fmax3(mx, s[rr], s[rr + 1]);
    mx = max_halves(mx);
    // online softmax update with the lazy reference of the prefill kernel:
    // the exponent reference m moves only when some row of the wave has
    // grown past it by more than kLazyLog2 (log2 units), so P <= 2^kLazyLog2
    // and O, l are rescaled only on those tiles.  A row that has seen no key
    // yet keeps m = -inf, l = 0, O = 0 (and takes alpha = 1 rather than
    // exp2(-inf - -inf)).  Where O lives in AGPRs (more than 256 registers a
    // wave) the multiply's operands are pinned to AGPRs on both sides (empty
    // asm, "a" constraint), which keeps the copy to vector registers inside
    // this rare branch.
    if (__any(mx > m_run + lazy)) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if constexpr (D >= 128) asm volatile("" : "+a"(o[db]));
        o[db] *= alpha;
        if constexpr (D >= 128) asm volatile("" : "+a"(o[db]));
      }
    }
    const float mc = m_run == -INFINITY ? 0.f : m_run * c;
    // P^T (bf16) as B operands: k-step ks covers keys 16 ks + 4 hi + 0..3 and
    // 16 ks + 8 + 4 hi + 0..3, registers 8 ks .. 8 ks + 7
    bf16x8 pb[2];
    float ls[4] = {-0.f, -0.f, -0.f, -0.f};  // x + -0 = x: the first adds fold away
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      u32x4 t;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float e0 = exp2_fast(__builtin_fmaf(s[8 * ks2 + 2 * h], c, -mc));
        const float e1 = exp2_fast(__builtin_fmaf(s[8 * ks2 + 2 * h + 1], c, -mc));
        t[h] = pack_bf16x2(e0, e1);
        ls[h] += e0 + e1;
      }
      pb[ks2] = __builtin_bit_cast(bf16x8, t);
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const i16x4 a0 = read_vt(vs, 16 * ks2 + 4 * hi, db);
        const i16x4 a1 = read_vt(vs, 16 * ks2 + 8 + 4 * hi, db);
        const u32x2 w0 = __builtin_bit_cast(u32x2, a0), w1 = __builtin_bit_cast(u32x2, a1);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
        o[db] = mfma_bf16_32x32x16(a, pb[ks2], o[db]);
      }
    // every read of this slot has returned before the slot is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(slot, i + 2);
  };

  issue(S0, 0);
  issue(S1, 1);
  // Every trip runs a step on slot 0, then one on slot 1, and an odd last
  // tile gets its own step after the loop.  So every read of a slot has
  // exactly one tile's loads (into the other slot) issued after it, in
  // program order as well as in the compiler's wait bookkeeping.
  int i = 0;
  for (; i + 1 < n_my; i += 2) {
    step(i, S0);
    step(i + 1, S1);
  }
  if (i < n_my) step(i, S0);

  // ---- merge the NW waves through LDS (slot 0 reused) ---------------------
  const float l_tot = sum_halves(l_run);
  wait_vmem<0>();   // the trailing zero loads into the ring have landed
  __syncthreads();  // and every wave has finished with its ring
  float* ml = reinterpret_cast<float*>(S0);  // [NW][64]: m of 32 rows, then l
  float* ob = ml + NW * 64;                   // [NW - 1][NDB * 16][64]: scaled O of waves 1..NW-1
  if (hi == 0) {
    ml[wave * 64 + l32] = m_run;
    ml[wave * 64 + 32 + l32] = l_tot;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = __builtin_fmaxf(M, ml[w * 64 + l32]);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float mw = ml[w * 64 + l32];
    L += mw == -INFINITY ? 0.f : ml[w * 64 + 32 + l32] * exp2_fast((mw - M) * c);
  }
  const float f = m_run == -INFINITY ? 0.f : exp2_fast((m_run - M) * c);
  if (wave > 0) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) ob[((wave - 1) * NDB * 16 + db * 16 + rr) * 64 + lane] = o[db][rr] * f;
  }
  __syncthreads();
  if (wave == 0 && rok) {
    const size_t g = row0 + (size_t)r;  // global query row in [B * Hq * Nq]
    const size_t rows = (size_t)p.B * p.Hq * Nq;
    const bool direct = p.splits == 1;
    float* orow = direct ? p.o + g * D : p.part_o + ((size_t)split * rows + g) * D;
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 4 * gq + e;
          float acc = o[db][rr] * f;
#pragma unroll
          for (int w = 1; w < NW; ++w) acc += ob[((w - 1) * NDB * 16 + db * 16 + rr) * 64 + lane];
          val[e] = acc * inv;
        }
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * gq + 4 * hi) = val;
      }
    if (hi == 0) {
      const float lse = L > 0.f ? M * p.scale + __logf(L) : -INFINITY;
      if (direct) p.lse[g] = lse;
      else p.part_lse[(size_t)split * rows + g] = lse;
    }
  }
}

// Combine the chunks of every query row: lse = ln sum_c exp(lse_c),
// O = sum_c exp(lse_c - lse) O_c (a chunk with lse_c = -inf saw no key of
// that row and weighs 0; a row with no key at all gets O = 0, lse = -inf).
// One pass with a running maximum, in blocks of U chunks whose lse and O
// loads are all issued together, so a row costs one memory round trip per
// U chunks.
template <int D>
__global__ __launch_bounds__(256) void dec_combine_kernel(DecBf16Params p) {
  constexpr int TPR = D / 4;      // threads per row, one float4 each
  constexpr int RPB = 256 / TPR;  // rows per workgroup
  constexpr int U = 8;
  const size_t rows = (size_t)p.B * p.Hq * p.Nq;
  const size_t g = (size_t)blockIdx.x * RPB + threadIdx.x / TPR;
  if (g >= rows) return;
  const int c4 = (int)threadIdx.x % TPR;
  const int S = p.splits;
  const float* pl = p.part_lse + g;
  const float* po = p.part_o + g * D + 4 * c4;
  float M = -INFINITY, W = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; s += U) {
    float l[U];
    f32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = s + u < S;
      l[u] = ok ? pl[(size_t)(s + u) * rows] : -INFINITY;
      x[u] = ok ? *reinterpret_cast<const f32x4*>(po + (size_t)(s + u) * rows * D) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mb = l[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mb = __builtin_fmaxf(mb, l[u]);
    const float mn = __builtin_fmaxf(M, mb);
    if (mn == -INFINITY) continue;  // nothing seen yet
    const float r = __expf(M - mn);  // 0 while M = -inf
    W *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = __expf(l[u] - mn);  // 0 for lse_c = -inf
      W += w;
      acc += w * x[u];
    }
    M = mn;
  }
  float* orow = p.o + g * D + 4 * c4;
  if (M == -INFINITY) {
    *reinterpret_cast<f32x4*>(orow) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c4 == 0) p.lse[g] = -INFINITY;
    return;
  }
  *reinterpret_cast<f32x4*>(orow) = acc * (1.f / W);
  if (c4 == 0) p.lse[g] = M + __logf(W);
}

template <int D, bool CAUSAL>
hipError_t launch(const DecBf16Params& p, hipStream_t stream) {
  const int R = (p.Hq / p.Hkv) * p.Nq;
  const unsigned grid = (unsigned)((R + 31) / 32) * (unsigned)p.splits * (unsigned)p.B * (unsigned)p.Hkv;
  hipLaunchKernelGGL((dec_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(DecCfg<D>::NW * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  constexpr int RPB = 256 / (D / 4);
  const size_t rows = (size_t)p.B * p.Hq * p.Nq;
  hipLaunchKernelGGL((dec_combine_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Device memory for the chunk partials of decode calls that bring no
// workspace (fa_fwd_bf16_decode_noalloc).  Each device the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address comes only from
// hipGetSymbolAddress with the device current (dec_scratch below).
static __device__ __align__(256) unsigned char scratch[kDecScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
}  // namespace

hipError_t dec_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* a = g_scratch[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    // once per device, with that device current; two threads racing here
    // look up and store the same address
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (a == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(a, std::memory_order_release);
  }
  *ptr = a;
  return hipSuccess;
}

hipError_t launch_dec_bf16(const DecBf16Params& p, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 64: return causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
    case 128: return causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
    case 256: return causal ? launch<256, true>(p, stream) : launch<256, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

int dec_bf16_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int requested, int num_cus) {
  const int ntile = (Nk + kTileKeys - 1) / kTileKeys;
  // s chunks of ceil(ntile / s) tiles may need fewer than s chunks to cover
  // every tile: return the number that is actually non-empty
  auto effective = [ntile](int s) {
    const int ct = (ntile + s - 1) / s;
    return (ntile + ct - 1) / ct;
  };
  if (requested >= 1) return effective(requested < ntile ? requested : ntile);

  // Cost model: every workgroup streams ct tiles of K and V at its share of
  // the HBM bandwidth, workgroups run in rounds of one per resident slot,
  // and more than one chunk adds the partial results' write and read plus
  // one more launch.  Ties go to fewer chunks.
  const int nw = d == 256 ? DecCfg<256>::NW : DecCfg<128>::NW;
  const double slots = (double)(num_cus > 0 ? num_cus : 1) * (d == 64 ? DecCfg<64>::MINB : 1);
  const int R = (Hq / Hkv) * Nq;
  const double units = (double)B * Hkv * ((R + 31) / 32);
  const double tile_bytes = (double)kTileKeys * d * 2 * 2;
  const double rows = (double)B * Hq * Nq;
  const double bw = 5e12, t_launch = 4e-6;
  int max_s = ntile / (2 * nw);  // at least two tiles per wave
  max_s = max_s < 1 ? 1 : (max_s > 256 ? 256 : max_s);
  int best = 1;
  double best_t = 0.0;
  for (int s = 1; s <= max_s; ++s) {
    if (effective(s) != s) continue;
    const int ct = (ntile + s - 1) / s;
    const double rounds = std::ceil(units * s / slots);
    double t = rounds * std::ceil((double)ct / nw) * nw * tile_bytes * slots / bw;
    if (s > 1) t += 2.0 * s * rows * (d + 1) * 4 / bw + t_launch;
    if (s == 1 || t < best_t * (1.0 - 1e-9)) {
      best_t = t;
      best = s;
    }
  }
  return best;
}

}  // namespace fa
