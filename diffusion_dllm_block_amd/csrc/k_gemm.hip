// Dense projections y = x . W^T of the transformer (QKV, output, gate/up, down, LM head)
// with their element-wise tails fused into the epilogue.
//
// Every kernel produces an fp32 tile of 128 "virtual" output columns in LDS and hands it
// to one epilogue (kernels.h: EpiKind):
//   QKV    : RoPE on q and k (rotate-half, pairs j and j + D/2, table cos/sin[pos][j]),
//            q scattered to [B][Hq][R][D], k into the cache K [B][Hkv][Sp][D], v into the
//            transposed, 32-key-blocked cache Vt (vt_off; the block's own K/V written in
//            place);
//   SWIGLU : a virtual tile is 64 gate rows + the matching 64 up rows of W, so the tile
//            holds both halves of silu(gate) * up;
//   RESID  : fp32 residual stream += tile;  F32: logits = logit_scale * tile;  STORE.
//
// Kernels:
//   gemm_skinny_bf16 (M <= 64): weight streaming, 64-column tiles of 8 waves (see below).
//     Residual GEMMs split K over gridDim.y and leave fp32 partials that the next
//     RMSNorm adds into the residual stream in split order; the others split K only
//     when the column tiles alone cannot fill the chip, and then the last workgroup of
//     a tile (device-scope arrival counter) sums the partials in split order and runs
//     the epilogue.  Deterministic either way: no float atomics.
//   gemm_tiled_bf16 (M > 64): 128x128 output tiles, 64-wide K stages double-buffered in
//     LDS with register prefetch, 4 waves each computing 64x64 with 32x32x16 MFMAs; the
//     same split-K schemes for shapes with too few tiles.
//   gemm_f32: SIMT fp32 kernel for fp32 models (32x128 tiles).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dllm {

template <int EPI>
__device__ __forceinline__ int wrow_of(int vc, int F) {
  if constexpr (EPI == EPI_SWIGLU) {
    int t = vc >> 7, j = vc & 127;
    return (j < 64) ? (t * 64 + j) : (F + t * 64 + (j - 64));
  } else {
    return vc;
  }
}

__device__ __forceinline__ float silu(float x) { return x / (1.f + expf(-x)); }
// SwiGLU output value of one row and column from its gate and up sums.
__device__ __forceinline__ uint16_t swiglu_bf16(float gt, float up) { return f2bf(silu(gt) * up); }

__device__ __forceinline__ int acc_row(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

// Element-by-element epilogue over an fp32 tile in LDS (tile[r * ldt + c] is output row
// m0 + r and virtual column vc0 + c, c < 128): the fallback of epilogue() for shapes or
// pointers that the 4-wide form does not cover.
template <typename T, int EPI>
__device__ void epilogue_scalar(const float* tile, int ldt, int rows, int m0, int vc0, int M, int Nv,
                         const EpiArgs& e) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if constexpr (EPI == EPI_STORE || EPI == EPI_F32 || EPI == EPI_RESID) {
    for (int i = tid; i < rows * 128; i += nt) {
      int r = i >> 7, c = i & 127;
      int m = m0 + r, vc = vc0 + c;
      if (m >= M || vc >= Nv) continue;
      float v = tile[r * ldt + c];
      int64_t o = (int64_t)m * e.ldy + vc;
      if constexpr (EPI == EPI_STORE) Elt<T>::store((T*)e.y, o, v);
      else if constexpr (EPI == EPI_F32) ((float*)e.y)[o] = v * e.scale;
      else ((float*)e.y)[o] += v;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int t = vc0 >> 7;
    for (int i = tid; i < rows * 64; i += nt) {
      int r = i >> 6, c = i & 63;
      int m = m0 + r, col = t * 64 + c;
      if (m >= M || col >= e.F) continue;
      float gt = tile[r * ldt + c], up = tile[r * ldt + 64 + c];
      Elt<T>::store((T*)e.y, (int64_t)m * e.F + col, silu(gt) * up);
    }
  } else {  // EPI_QKV
    const int D = e.D, half = D >> 1;
    const bool vtile = vc0 >= (e.Hq + e.Hkv) * D;
    for (int i = tid; i < rows * 64; i += nt) {
      int r, pidx;
      if (vtile) { pidx = i / rows; r = i % rows; }   // consecutive threads: consecutive positions
      else { r = i >> 6; pidx = i & 63; }              // consecutive threads: consecutive dims
      int m = m0 + r;
      int hh = pidx / half, j = pidx % half;
      int ca = hh * D + j;
      int vca = vc0 + ca;
      if (m >= M || vca >= Nv) continue;
      float x1 = tile[r * ldt + ca], x2 = tile[r * ldt + ca + half];
      int bs = m / e.R, ri = m % e.R, pos = e.pos0 + ri;
      int gh = vca / D;
      if (gh < e.Hq + e.Hkv) {
        float cs = e.rcos[(int64_t)pos * half + j], sn = e.rsin[(int64_t)pos * half + j];
        float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
        T* dst;
        if (gh < e.Hq) dst = (T*)e.qo + (((int64_t)bs * e.Hq + gh) * e.R + ri) * D;
        else dst = (T*)e.kc + (((int64_t)bs * e.Hkv + (gh - e.Hq)) * e.Sp + pos) * D;
        Elt<T>::store(dst, j, y1);
        Elt<T>::store(dst, j + half, y2);
      } else {
        int h = gh - e.Hq - e.Hkv;
        T* dst = (T*)e.vtc + ((int64_t)bs * e.Hkv + h) * D * (int64_t)e.Sp;
        Elt<T>::store(dst, vt_off(j, pos, D), x1);
        Elt<T>::store(dst, vt_off(j + half, pos, D), x2);
      }
    }
  }
}

// 4 adjacent outputs: 8 bytes of bf16 or 16 bytes of fp32 (callers check the alignment).
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<u16x4*>(p) = u16x4{f2bf(a), f2bf(b), f2bf(c), f2bf(d)};
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
}
__device__ __forceinline__ bool aligned_to(const void* p, int bytes) {
  return ((uintptr_t)p & (uintptr_t)(bytes - 1)) == 0;
}
__device__ __forceinline__ int ilog2(int v) { return 31 - __builtin_clz(v); }

// Epilogue over an fp32 tile in LDS: tile[r * ldt + c] is output row m0 + r and virtual
// column vc0 + c (c < 128); ldt % 4 == 0 and the tile 16-byte aligned.  Each thread takes
// 4 adjacent outputs (16-byte LDS reads, one 8- or 16-byte store) and works out a row's
// sequence and position once per row; V is written 4 positions at a time.  Shapes or
// pointers outside that form go through epilogue_scalar (same arithmetic per element).
template <typename T, int EPI>
__device__ void epilogue(const float* tile, int ldt, int rows, int m0, int vc0, int M, int Nv,
                         const EpiArgs& e) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if constexpr (EPI == EPI_STORE || EPI == EPI_F32 || EPI == EPI_RESID) {
    using O = typename std::conditional<EPI == EPI_STORE, T, float>::type;
    O* y = (O*)e.y;
    const bool vec = e.ldy % 4 == 0 && aligned_to(y, 4 * (int)sizeof(O));
    for (int i = tid; i < rows * 32; i += nt) {
      const int r = i >> 5, c = 4 * (i & 31);
      const int m = m0 + r, vc = vc0 + c;
      if (m >= M || vc >= Nv) continue;
      const float4 v = *reinterpret_cast<const float4*>(tile + r * ldt + c);
      O* p = y + (int64_t)m * e.ldy + vc;
      if (vec && vc + 3 < Nv) {
        if constexpr (EPI == EPI_STORE) {
          store4<O>(p, v.x, v.y, v.z, v.w);
        } else if constexpr (EPI == EPI_F32) {
          store4<float>(p, v.x * e.scale, v.y * e.scale, v.z * e.scale, v.w * e.scale);
        } else {
          float4 o = *reinterpret_cast<const float4*>(p);
          o.x += v.x; o.y += v.y; o.z += v.z; o.w += v.w;
          *reinterpret_cast<float4*>(p) = o;
        }
      } else {
        const float vv[4] = {v.x, v.y, v.z, v.w};
        for (int u = 0; u < 4 && vc + u < Nv; ++u) {
          if constexpr (EPI == EPI_STORE) Elt<O>::store(p, u, vv[u]);
          else if constexpr (EPI == EPI_F32) p[u] = vv[u] * e.scale;
          else p[u] += vv[u];
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int t = vc0 >> 7;
    T* y = (T*)e.y;
    if (e.F % 4 != 0 || !aligned_to(y, 4 * (int)sizeof(T))) {
      epilogue_scalar<T, EPI>(tile, ldt, rows, m0, vc0, M, Nv, e);
      return;
    }
    for (int i = tid; i < rows * 16; i += nt) {
      const int r = i >> 4, c = 4 * (i & 15);
      const int m = m0 + r, col = t * 64 + c;
      if (m >= M || col >= e.F) continue;
      const float4 gt = *reinterpret_cast<const float4*>(tile + r * ldt + c);
      const float4 up = *reinterpret_cast<const float4*>(tile + r * ldt + 64 + c);
      store4<T>(y + (int64_t)m * e.F + col, silu(gt.x) * up.x, silu(gt.y) * up.y,
                silu(gt.z) * up.z, silu(gt.w) * up.w);
    }
  } else {  // EPI_QKV
    const int D = e.D, half = D >> 1;
    const int ab = 4 * (int)sizeof(T);
    const bool vec = D >= 8 && (D & (D - 1)) == 0 && D <= 128 && rows >= 4 &&
                     (rows & (rows - 1)) == 0 && aligned_to(e.qo, ab) &&
                     aligned_to(e.kc, ab) && aligned_to(e.vtc, ab) && aligned_to(e.rcos, 16) &&
                     aligned_to(e.rsin, 16);
    if (!vec) {
      epilogue_scalar<T, EPI>(tile, ldt, rows, m0, vc0, M, Nv, e);
      return;
    }
    const int nqk = e.Hq + e.Hkv, lgD = ilog2(D);
    // whole runs of 4 positions in one sequence and one 32-key block of the value cache
    const bool v4 = e.R % 4 == 0 && e.pos0 % 4 == 0;
    for (int cb = 0; cb < 128; cb += D) {  // the heads of the tile, D columns each
      const int gh = (vc0 + cb) >> lgD;
      if (vc0 + cb >= Nv) break;
      if (gh < nqk) {
        // q or k head: RoPE pairs (j, j + D/2), 4 adjacent j per thread
        const int lgg = lgD - 3;  // log2 of the 4-wide groups per half (D/8)
        for (int i = tid; i < (rows << lgg); i += nt) {
          const int r = i >> lgg, j = 4 * (i & ((1 << lgg) - 1));
          const int m = m0 + r;
          if (m >= M) continue;
          const int bs = m / e.R, ri = m - bs * e.R, pos = e.pos0 + ri;
          const float4 x1 = *reinterpret_cast<const float4*>(tile + r * ldt + cb + j);
          const float4 x2 = *reinterpret_cast<const float4*>(tile + r * ldt + cb + half + j);
          const float4 cs = *reinterpret_cast<const float4*>(e.rcos + (int64_t)pos * half + j);
          const float4 sn = *reinterpret_cast<const float4*>(e.rsin + (int64_t)pos * half + j);
          T* dst;
          if (gh < e.Hq) dst = (T*)e.qo + (((int64_t)bs * e.Hq + gh) * e.R + ri) * D;
          else dst = (T*)e.kc + (((int64_t)bs * e.Hkv + (gh - e.Hq)) * e.Sp + pos) * D;
          store4<T>(dst + j, x1.x * cs.x - x2.x * sn.x, x1.y * cs.y - x2.y * sn.y,
                    x1.z * cs.z - x2.z * sn.z, x1.w * cs.w - x2.w * sn.w);
          store4<T>(dst + j + half, x2.x * cs.x + x1.x * sn.x, x2.y * cs.y + x1.y * sn.y,
                    x2.z * cs.z + x1.z * sn.z, x2.w * cs.w + x1.w * sn.w);
        }
      } else {
        // value head: transposed, 32-key-blocked cache; consecutive threads take
        // consecutive runs of 4 positions of one dim
        const int h = gh - nqk;
        const int lgn = ilog2(rows) - 2;  // log2 of the runs of 4 rows
        for (int i = tid; i < (rows >> 2) * D; i += nt) {
          const int d = i >> lgn, r = 4 * (i & ((1 << lgn) - 1));
          const int m = m0 + r;
          if (m >= M) continue;
          if (v4 && m + 3 < M) {
            const int bs = m / e.R, ri = m - bs * e.R, pos = e.pos0 + ri;
            T* dst = (T*)e.vtc + ((int64_t)bs * e.Hkv + h) * D * (int64_t)e.Sp;
            store4<T>(dst + vt_off(d, pos, D), tile[r * ldt + cb + d],
                      tile[(r + 1) * ldt + cb + d], tile[(r + 2) * ldt + cb + d],
                      tile[(r + 3) * ldt + cb + d]);
          } else {
            for (int u = 0; u < 4 && m + u < M; ++u) {
              const int mu = m + u, bs = mu / e.R, pos = e.pos0 + (mu - bs * e.R);
              T* dst = (T*)e.vtc + ((int64_t)bs * e.Hkv + h) * D * (int64_t)e.Sp;
              Elt<T>::store(dst, vt_off(d, pos, D), tile[(r + u) * ldt + cb + d]);
            }
          }
        }
      }
    }
  }
}

// Sum of `splits` device-coherent partials p[0], p[stride], ... in split order; the
// loads of a group of 8 are issued together.
__device__ __forceinline__ float sum_splits(const float* p, int64_t stride, int splits) {
  float s = 0.f;
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (s0 + u < splits) ? ld_dev(p + (s0 + u) * stride) : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  return s;
}

// Sum split-K partials [splits][M][Nv] of one 128-column tile in split order into LDS.
__device__ __forceinline__ void gather_partials(float* tile, int ldt, int rows, int m0, int vc0,
                                                int M, int Nv, int splits, const float* part) {
  for (int i = threadIdx.x; i < rows * 128; i += blockDim.x) {
    int r = i >> 7, c = i & 127;
    int m = m0 + r, vc = vc0 + c;
    tile[r * ldt + c] = (m < M && vc < Nv)
        ? sum_splits(part + (int64_t)m * Nv + vc, (int64_t)M * Nv, splits) : 0.f;
  }
}

// ============================================================================
// skinny bf16 GEMM (M <= 64): weight streaming
// ============================================================================
// virtual column -> weight row for 64-column tiles:
//   SWIGLU: tile t = gate rows 32t..+32 then up rows F+32t..+32;
//   QKV (head_dim 128): tile t = head t/2, dims 32(t&1)..+32 then the same dims + 64,
//   so RoPE pairs (d, d+64) sit in one tile.
template <int EPI>
__device__ __forceinline__ int wrow_s2(int vc, int F) {
  const int t = vc >> 6, c = vc & 63;
  if constexpr (EPI == EPI_SWIGLU) {
    return c < 32 ? t * 32 + c : F + t * 32 + (c - 32);
  } else if constexpr (EPI == EPI_QKV) {
    const int hs = t >> 1, part = t & 1;
    return hs * 128 + (c < 32 ? part * 32 + c : 64 + part * 32 + (c - 32));
  } else {
    return vc;
  }
}

// Persistent weight-streaming GEMM for M <= 64 rows.
//   * One 8-wave workgroup per CU, pinned to one K range of KW = 8 * KS
//     (blockIdx % splits); its activation slice X[M][KW] is loaded into LDS once.
//   * The workgroup walks 16-column groups (wid, wid + nw, ...).  For a group, wave w
//     covers the K sub-range [w KS, (w+1) KS) with 16x16x32 MFMAs; the 8 partial sums
//     are added in LDS in wave order, and each of the MT*4 result rows of 64 lanes is
//     written as one 256-byte store (blocked partial layout, PartView in kernels.h).  So
//     a wave keeps only KS/32 loads per lane in flight (a modest, steady stream per CU)
//     while the partials written per group are those of one K range of KW.
//   * Register t is refilled with the next group's weights right after the MFMAs of
//     step t consumed it.  After the last group the refills read one fixed cached line
//     instead of branching: no data-dependent branches, so the wait counts stay exact.
//   * Partials (virtual column order) are summed in split order by reduce_epilogue, or
//     for the residual GEMMs by the next RMSNorm.  They go out as device-coherent
//     (written-through) stores: the next kernel reads them from every XCD, and the
//     8B cached step measured 4.199 -> 4.185 ms with them (bit-identical).
template <int MT, int KS> struct SkinnyCfg {
  static constexpr int KW = 8 * KS;                  // K range of a workgroup
  static constexpr int NLOAD = KS / 32;              // weight loads per lane per group
  static constexpr int LDX = KW + 8;                 // LDS row stride (elements)
  static constexpr int SLOTS = MT * 4;               // result rows of 64 lanes per group
  // the cross-wave sums go through LDS at most 8 result rows at a time, which leaves
  // room for a 128-deep per-wave K range at 64 rows (64 x 24576 x 4096: 67.8 -> 48.6 us
  // against a 64-deep one, whose 2 loads per lane in flight starved the weight stream)
  static constexpr int RS = SLOTS < 8 ? SLOTS : 8;
  static_assert(MT * 16 * LDX * 2 + 8 * RS * 64 * 4 <= 160 * 1024, "LDS budget");
};

template <int MAP, int MT, int KS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_skinny_bf16(
    const uint16_t* __restrict__ X, int ldx, const uint16_t* __restrict__ W, int M, int Nv,
    int K, int F, int splits, int ngrp, float* __restrict__ part) {
  using C = SkinnyCfg<MT, KS>;
  __shared__ __attribute__((aligned(16))) uint16_t Xs[MT * 16 * C::LDX];
  __shared__ __attribute__((aligned(16))) float red[8][C::RS][64];
  const int split = blockIdx.x % splits;
  const int wid = blockIdx.x / splits;
  const int nw = gridDim.x / splits;  // workgroups per K range (grid is a multiple of splits)
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, ln = l & 15, g = l >> 4;
  const int kw0 = split * C::KW;      // the workgroup's K range
  const int ks0 = kw0 + w * KS;       // this wave's K sub-range

  auto wptr = [&](int grp) {  // columns past Nv read a clamped valid row (never used)
    const int vc = min(grp * 16 + ln, Nv - 1);
    return W + (int64_t)wrow_s2<MAP>(vc, F) * K + ks0 + 8 * g;
  };
  u32x4 wr[C::NLOAD];
  {
    // activation slice -> LDS by direct global->LDS loads (rows >= M read row M-1; their
    // outputs are never used).  Load slot s fills LDS bytes [1024 s, 1024 s + 1024) of
    // the padded slice, lane l its 16-byte chunk q = 64 s + l: row q / RC, chunk q % RC
    // of that row, where chunk RC - 1 is the row's pad (it loads an in-row chunk, never
    // read).  The first group's weight loads follow in t order, like the refills in the
    // loop, and the wait before the barrier leaves just them in flight, so the weight
    // stream's first HBM round trip overlaps the staging and the loop's wait counts are
    // the same on entry and on the back edge.
    constexpr int RC = C::LDX / 8;            // 16-byte chunks per LDS row, pad included
    constexpr int NCH = MT * 16 * RC;         // chunks in the slice
    constexpr int NSLOT = (NCH + 63) / 64;    // 1 KB load slots
    unsigned char* xsb = reinterpret_cast<unsigned char*>(Xs);
#pragma unroll
    for (int it = 0; it < (NSLOT + 7) / 8; ++it) {
      const int slot = it * 8 + w;
      if (slot < NSLOT) {  // uniform over the wave
        const int q = slot * 64 + l;
        const int r = q / RC, cc = q % RC;
        const uint16_t* src =
            X + (int64_t)min(r, M - 1) * ldx + kw0 + 8 * min(cc, RC - 2);
        if (q < NCH)
          __builtin_amdgcn_global_load_lds(
              (const __attribute__((address_space(1))) void*)src,
              (__attribute__((address_space(3))) void*)(xsb + slot * 1024), 16, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* wp = wptr(min(wid, ngrp - 1));
#pragma unroll
    for (int t = 0; t < C::NLOAD; ++t) {
      wr[t] = *reinterpret_cast<const u32x4*>(wp + 32 * t);
      __builtin_amdgcn_sched_barrier(0);
    }
    // this wave's slice loads have landed once only the NLOAD weight loads are in flight
    __builtin_amdgcn_s_waitcnt((C::NLOAD & 15) | ((C::NLOAD >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
  }
  __syncthreads();

  // A do-while with no exit between the loads above and the loop: an exit branch here
  // lets the compiler sink the first weight loads below the barrier.  The host launches
  // at most ngrp workgroups per K range, so wid < ngrp; the partial store is guarded
  // anyway (uniform over the workgroup).
  const uint16_t* xs = &Xs[ln * C::LDX + w * KS + 8 * g];
  int grp = wid;
  do {
    const bool has_next = grp + nw < ngrp;
    // refill source: the next group, or (after the last group) this wave's first weight
    // line, which stays cached; the same offsets keep the loads' addresses immediate
    const uint16_t* wpn = has_next ? wptr(grp + nw) : W + ks0 + 8 * g;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{};
#pragma unroll
    for (int t = 0; t < C::NLOAD; ++t) {
      u32x4 a[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        a[mt] = *reinterpret_cast<const u32x4*>(xs + mt * 16 * C::LDX + 32 * t);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16(as_bf16x8(a[mt]), as_bf16x8(wr[t]), acc[mt]);
      wr[t] = *reinterpret_cast<const u32x4*>(wpn + 32 * t);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane (column ln, group g) holds rows mt*16 + 4g + r: slot mt*4 + r; the slots go
    // through LDS RS at a time
#pragma unroll
    for (int h = 0; h < C::SLOTS / C::RS; ++h) {
      if (h > 0) __syncthreads();  // red is rewritten by the next slots
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mt * 4 + r >= h * C::RS && mt * 4 + r < (h + 1) * C::RS)
            red[w][mt * 4 + r - h * C::RS][l] = acc[mt][r];
      __syncthreads();
      if (grp < ngrp) {
        float* blk = part + ((int64_t)split * ngrp + grp) * (MT * 16 * 16);
        for (int sl = w; sl < C::RS; sl += 8) {
          float v = red[0][sl][l];
#pragma unroll
          for (int ww = 1; ww < 8; ++ww) v += red[ww][sl][l];
          st_dev(&blk[(h * C::RS + sl) * 64 + l], v);
        }
      }
    }
    __syncthreads();  // red is rewritten by the next group
    grp += nw;
  } while (grp < ngrp);
}

// ============================================================================
// tiled bf16 GEMM
// ============================================================================
constexpr int TL = 132;  // LDS row stride of the fp32 128-column epilogue tile
constexpr int TB_K = 64;
constexpr int TB_LD = TB_K + 8;
constexpr int TB_AB_BYTES = 2 * 2 * 128 * TB_LD * 2;
constexpr int TB_TILE_BYTES = 128 * TL * 4;
constexpr int TB_SMEM = TB_AB_BYTES > TB_TILE_BYTES ? TB_AB_BYTES : TB_TILE_BYTES;

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_tiled_bf16(
    const uint16_t* __restrict__ X, int ldx, const uint16_t* __restrict__ W, int M, int Nv, int K,
    int kchunk, int splits, float* part, int* counters, EpiArgs e, int tn0) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[TB_SMEM];
  __shared__ int flag;
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + 2 * 128 * TB_LD;
  float* tile = reinterpret_cast<float*>(smem);
  // row tiles fastest: the row tiles of one weight tile are dispatched together, so the
  // weight tile streams from HBM once and the others find it in the Infinity Cache
  const int tm = blockIdx.x, tn = tn0 + blockIdx.y, split = blockIdx.z;
  const int m0 = tm * 128, vc0 = tn * 128;
  const int tid = threadIdx.x;
  const int w = tid >> 6, wm = w >> 1, wn = w & 1, l = tid & 63, lr = l & 31, g = l >> 5;
  const int kb = split * kchunk;
  const int ke = min(K, kb + kchunk);
  const int nst = (ke - kb) / TB_K;

  // loader: element e = tid + 256 i  ->  row e >> 3, 16-byte column e & 7
  // rows past M / columns past Nv load from a clamped valid address; their results are
  // discarded by the epilogue (unconditional loads keep the load counting exact)
  const uint16_t* arow[4];
  const uint16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int ee = tid + 256 * i;
    int r = ee >> 3, c8 = ee & 7;
    int m = min(m0 + r, M - 1), vc = min(vc0 + r, Nv - 1);
    arow[i] = X + (int64_t)m * ldx + kb + 8 * c8;
    brow[i] = W + (int64_t)wrow_of<EPI>(vc, e.F) * K + kb + 8 * c8;
  }
  // two register sets: the global loads of stage s + 2 are issued before stage s is
  // computed, so they have two compute phases to arrive
  u32x4 ra[2][4], rb[2][4];
  auto load = [&](int set, int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[set][i] = *reinterpret_cast<const u32x4*>(arow[i] + st * TB_K);
      rb[set][i] = *reinterpret_cast<const u32x4*>(brow[i] + st * TB_K);
    }
  };
  auto store = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int ee = tid + 256 * i;
      int r = ee >> 3, c8 = ee & 7;
      *reinterpret_cast<u32x4*>(&As[(buf * 128 + r) * TB_LD + 8 * c8]) = ra[set][i];
      *reinterpret_cast<u32x4*>(&Bs[(buf * 128 + r) * TB_LD + 8 * c8]) = rb[set][i];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < TB_K / 16; ++kk) {
      u32x4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(&As[(buf * 128 + wm * 64 + i * 32 + lr) * TB_LD + 16 * kk + 8 * g]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const u32x4*>(&Bs[(buf * 128 + wn * 64 + j * 32 + lr) * TB_LD + 16 * kk + 8 * g]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(as_bf16x8(a[i]), as_bf16x8(b[j]), acc[i][j]);
    }
  };

  // stage s lives in LDS buffer s & 1 and register set s & 1
  load(0, 0);
  store(0, 0);
  if (nst > 1) load(1, 1);
  __syncthreads();
  // pairs of stages (one loop latch: the accumulators keep their registers)
  int st = 0;
  for (; st + 1 < nst; st += 2) {
    if (st + 2 < nst) load(0, st + 2);
    compute(0);
    store(1, 1);
    __syncthreads();
    if (st + 3 < nst) load(1, st + 3);
    compute(1);
    if (st + 2 < nst) store(0, 0);
    __syncthreads();
  }
  if (st < nst) {  // odd stage count: the last stage is in buffer 0
    compute(0);
    __syncthreads();  // the epilogue tile below reuses the operand buffers
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        tile[(wm * 64 + i * 32 + acc_row(v, g)) * TL + wn * 64 + j * 32 + lr] = acc[i][j][v];
  __syncthreads();
  if (splits == 1) {
    epilogue<uint16_t, EPI>(tile, TL, 128, m0, vc0, M, Nv, e);
    return;
  }
  if constexpr (EPI == EPI_RESID) {
    // deferred: the consumer of the residual stream sums the split partials in order
    for (int i = tid; i < 128 * 128; i += 256) {
      int r = i >> 7, c = i & 127;
      int m = m0 + r, vc = vc0 + c;
      if (m < M && vc < Nv) part[((int64_t)split * M + m) * Nv + vc] = tile[r * TL + c];
    }
    return;
  }
  for (int i = tid; i < 128 * 128; i += 256) {
    int r = i >> 7, c = i & 127;
    int m = m0 + r, vc = vc0 + c;
    if (m < M && vc < Nv) st_dev(&part[((int64_t)split * M + m) * Nv + vc], tile[r * TL + c]);
  }
  if (!arrive_last(&counters[tm * gridDim.y + blockIdx.y], splits, &flag)) return;
  gather_partials(tile, TL, 128, m0, vc0, M, Nv, splits, part);
  __syncthreads();
  epilogue<uint16_t, EPI>(tile, TL, 128, m0, vc0, M, Nv, e);
}

// ============================================================================
// large bf16 GEMM (M >= 512, the refresh): 256x256 output tiles, 8 waves (two per
// SIMD, so one can issue MFMAs while the other waits) each computing 128 rows x 64
// columns with 32x32x16 MFMAs.  K advances in stages of DK columns held in a ring of
// NSTG LDS slots filled by direct global->LDS loads (no staging registers), and the
// LDS operands of step kk + 1 are read while step kk is in the MFMAs.  The one barrier
// per stage comes before the stage's last k-step, whose MFMAs then cover the refill of
// the freed slot and the next stage's first operand reads (with the barrier at the
// stage boundary: 8B refresh 29.66 -> 29.44 ms, 7B 105.6 -> 103.7 ms; bit-identical, the
// products are summed in the same order).  The epilogue runs one 128x128
// quarter at a time through an fp32 LDS tile (the 128-column virtual tiles of the
// other kernels).  Residual GEMMs with too few tiles split K and leave fp32 partials
// [split][M][Nv] for the next RMSNorm.
// ============================================================================
constexpr int BG_T = 256;                                   // output tile (rows = cols)
constexpr int BG_THREADS = 512;
constexpr int BG_DK = 64, BG_NSTG = 2;                      // K per stage, ring slots
static_assert(BG_NSTG <= 4, "the wait counts cover at most two stages in flight");
constexpr int BG_AB_BYTES = BG_NSTG * 2 * BG_T * BG_DK * 2;  // ring of A and B stages
constexpr int BG_TILE_BYTES = 2 * 128 * TL * 4;             // two 128x128 quarters, fp32
constexpr int BG_SMEM = BG_AB_BYTES > BG_TILE_BYTES ? BG_AB_BYTES : BG_TILE_BYTES;
static_assert(BG_SMEM <= 160 * 1024, "LDS budget");

// Column tiles tn0 + blockIdx.x.  With splits > 1 the tile's K piece is stored as fp32
// partials [split][M][Nv - vbase] at column vc - vbase.
template <int EPI, int DK, int NSTG>
__global__ __launch_bounds__(BG_THREADS, 1) void gemm_big_bf16(
    const uint16_t* __restrict__ X, int ldx, const uint16_t* __restrict__ W, int M, int Nv, int K,
    int kchunk, int splits, float* part, EpiArgs e, int tn0, int vbase) {
  extern __shared__ __attribute__((aligned(16))) unsigned char bg_smem[];
  float* tile = reinterpret_cast<float*>(bg_smem);
  const int tn = tn0 + blockIdx.x, tm = blockIdx.y, split = blockIdx.z;
  const int m0 = tm * BG_T, vc0 = tn * BG_T;
  constexpr int WV = BG_THREADS / 64;          // waves: two row halves x 4 column groups
  constexpr int NT = BG_THREADS;
  constexpr int NJ = 16 / WV;                  // 32-column MFMA tiles per wave
  constexpr int WC = 32 * NJ;                  // columns per wave
  constexpr int RW = BG_T / WV;                // A (and B) tile rows each wave loads
  const int tid = threadIdx.x;
  // wave w: rows 128 (w & 1) .. +128, columns WC (w >> 1) .. +WC
  const int w = tid >> 6, wm = w & 1, wn = w >> 1, l = tid & 63, lr = l & 31, g = l >> 5;
  const int kb = split * kchunk;
  const int ke = min(K, kb + kchunk);

  // K stages of DK columns in a ring of NSTG LDS slots, filled by direct global->LDS
  // loads (no staging registers): each wave issues CPR/2 16-byte-per-lane loads of A
  // and of B per stage, each writing 1 KB of LDS (64 / CPR tile rows).  Rows are stored
  // unpadded with the 16-byte chunks XOR-swizzled by row (the mid kernel's layout note),
  // so the MFMA operand reads (32 rows at one k offset) are free of bank conflicts.
  constexpr int CPR = DK / 8;                  // 16-byte chunks per tile row
  constexpr int RPI = 64 / CPR;                // tile rows per load instruction
  constexpr int NI = RW / RPI;                 // load instructions per wave per matrix
  constexpr int HALF = BG_T * DK * 2;          // A (or B) bytes per stage
  constexpr int STG = 2 * HALF;
  const int nst = (ke - kb) / DK;
  auto swz = [](int r) { return CPR == 4 ? ((r >> 2) & 3) : ((r >> 1) & (CPR - 1)); };
  const uint16_t* asrc[NI];
  const uint16_t* bsrc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = w * RW + i * RPI + l / CPR;
    const int c = (l % CPR) ^ swz(row);
    asrc[i] = X + (int64_t)min(m0 + row, M - 1) * ldx + kb + c * 8;
    bsrc[i] = W + (int64_t)wrow_of<EPI>(min(vc0 + row, Nv - 1), e.F) * K + kb + c * 8;
  }
  auto issue = [&](int st) {
    unsigned char* base = bg_smem + (st % NSTG) * STG;
    st = min(st, nst - 1);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(asrc[i] + st * DK),
          (__attribute__((address_space(3))) void*)(base + (w * RW + i * RPI) * (DK * 2)), 16,
          0, 0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(bsrc[i] + st * DK),
          (__attribute__((address_space(3))) void*)(base + HALF + (w * RW + i * RPI) * (DK * 2)),
          16, 0, 0);
    }
  };
  f32x16 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  auto frag = [&](int slot, int kk, u32x4* a, u32x4* b) {
    const unsigned char* base = bg_smem + slot * STG;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + lr, c = 2 * kk + g;
      a[i] = *reinterpret_cast<const u32x4*>(base + r * (DK * 2) + ((c ^ swz(r)) * 16));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = wn * WC + j * 32 + lr, c = 2 * kk + g;
      b[j] = *reinterpret_cast<const u32x4*>(base + HALF + r * (DK * 2) + ((c ^ swz(r)) * 16));
    }
  };
  auto mfmas = [&](const u32x4* a, const u32x4* b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(as_bf16x8(a[i]), as_bf16x8(b[j]), acc[i][j]);
  };
  constexpr int NK = DK / 16;              // 16-deep k-steps per stage
  static_assert(NK % 2 == 0, "operand register sets alternate within and across stages");
  constexpr int RD = 4 + NJ, MF = 4 * NJ;  // operand reads and MFMAs per k-step
  constexpr int NL = 2 * NI;               // loads per wave per stage
  // s_waitcnt on vmcnt = n alone, and on vmcnt = n with lgkmcnt = 0
#define DLLM_VMWAIT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define DLLM_VMLGKWAIT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))
  // Every stage s lives in slot s % NSTG.  The prologue fills every slot; afterwards
  // each barrier (one per stage, taken one k-step before the stage ends, once every
  // wave holds the stage's last operands in registers) frees the stage's slot and
  // refills it NSTG stages ahead, and the last k-step's MFMAs run alongside those loads
  // and the next stage's first operand reads, so the barrier does not leave the MFMA
  // units waiting on LDS latency.  Loads past the last stage re-read it into a slot
  // that is never read, so that every barrier leaves NSTG - 2 later stages in flight.
  for (int s = 0; s < NSTG; ++s) issue(s);
  if constexpr (NSTG == 4) DLLM_VMWAIT(3 * NL);
  else if constexpr (NSTG == 3) DLLM_VMWAIT(2 * NL);
  else DLLM_VMWAIT(NL);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  u32x4 a[2][4], b[2][NJ];
  // k-steps 0 .. NK - 2 of the stage in `slot`, the operands of step 0 already in set 0
  auto body = [&](int slot) {
#pragma unroll
    for (int kk = 0; kk < NK - 1; ++kk) {
      frag(slot, kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
      mfmas(a[kk & 1], b[kk & 1]);
    }
    // Pin the issue order: the next step's reads alternate with this step's MFMAs.
    // Left alone, the scheduler reuses one operand register set and waits for every
    // read before each MFMA group.
#pragma unroll
    for (int kk = 0; kk < NK - 1; ++kk) {
#pragma unroll
      for (int i = 0; i < RD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 0x008: MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 0x100: LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, MF - RD, 0);
    }
  };
  frag(0, 0, a[0], b[0]);
  for (int st = 0; st + 1 < nst; ++st) {
    const int slot = st % NSTG;
    body(slot);
    // this wave's reads of the slot are done and stage st + 1 has landed (NSTG - 2
    // later stages may still be in flight); the barrier covers every wave's
    if constexpr (NSTG == 4) DLLM_VMLGKWAIT(2 * NL);
    else if constexpr (NSTG == 3) DLLM_VMLGKWAIT(NL);
    else DLLM_VMLGKWAIT(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(st + NSTG);  // into the slot just freed
    frag((st + 1) % NSTG, 0, a[0], b[0]);
    mfmas(a[1], b[1]);
    // the next stage's first reads early among the MFMAs, the loads spread over them
    static_assert(NL <= MF && MF % NL == 0 && RD <= MF, "one VMEM slot per MF / NL MFMAs");
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i % (MF / NL) == 0) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
    }
  }
  body((nst - 1) % NSTG);
  mfmas(a[1], b[1]);
  DLLM_VMWAIT(0);  // loads past the last stage land before the epilogue reuses the LDS
#undef DLLM_VMWAIT
#undef DLLM_VMLGKWAIT
  __syncthreads();  // the epilogue tile below reuses the operand slots

  // epilogue in two halves of 128 rows: the four waves of a half stage its two 128x128
  // quarters side by side in LDS, then every thread works through them
  for (int qm = 0; qm < 2; ++qm) {
    if (wm == qm) {
      float* t = tile + (wn * WC / 128) * 128 * TL;
      const int c0 = (wn * WC) % 128;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            t[(i * 32 + acc_row(v, g)) * TL + c0 + j * 32 + lr] = acc[i][j][v];
    }
    __syncthreads();
    const int pm0 = m0 + 128 * qm;
    for (int qn = 0; qn < 2; ++qn) {
      const float* t = tile + qn * 128 * TL;
      const int pvc0 = vc0 + 128 * qn;
      if (splits == 1) {
        epilogue<uint16_t, EPI>(t, TL, 128, pm0, pvc0, M, Nv, e);
      } else {
        // split over K: partials summed in split order by the next RMSNorm (residual
        // GEMMs) or by reduce_epilogue (a split tail of tiles), 4 columns per store
        const int Np = Nv - vbase;
        const bool vec = Np % 4 == 0;
        for (int i = tid; i < 128 * 32; i += NT) {
          const int r = i >> 5, c = 4 * (i & 31);
          const int m = pm0 + r, vc = pvc0 + c;
          if (m >= M || vc >= Nv) continue;
          float* dst = part + ((int64_t)split * M + m) * Np + (vc - vbase);
          const float4 v = *reinterpret_cast<const float4*>(t + r * TL + c);
          if (vec && vc + 3 < Nv) {
            *reinterpret_cast<float4*>(dst) = v;
          } else {
            const float vv[4] = {v.x, v.y, v.z, v.w};
            for (int u = 0; u < 4 && vc + u < Nv; ++u) dst[u] = vv[u];
          }
        }
      }
    }
    __syncthreads();
  }
}

// ============================================================================
// mid-size bf16 GEMM (kSkinnyRows < M <= 256: a batch of block steps, or the block and
// suffix rows of a prefix-mode step)
// ============================================================================
// One 256-row tile covers every row, so each weight tile is read once.  Output tiles are
// 128 virtual columns wide (the 64-column virtual order of wrow_s2, so split partials
// go through reduce_epilogue unchanged).  8 waves, 4 (rows) x 2 (columns), each 64 x 64
// with 2 x 2 32x32x16 MFMAs; K stages of 64 in a ring of three LDS slots filled by direct
// global->LDS loads two stages ahead; one barrier per stage.
// Work units, walked persistently by at most one workgroup per CU:
//   * units [0, ndp): whole tiles 0 .. ndp-1, full K, epilogue from an LDS tile;
//   * then every tile t >= ndp in `splits` K pieces of kst stages: fp32 partials
//     [split][M][Nv - 128 ndp], summed in split order by reduce_epilogue (or, residual
//     GEMMs, by the next RMSNorm).
// The plan splits everything for the residual and QKV GEMMs and, for the others, only the
// ragged last round of tiles, so the chip stays busy without a partial round trip for
// the bulk of the work.
// Split partials and the SwiGLU outputs leave as device-coherent (written-through) stores,
// which the next kernel reads from every XCD: bit-identical, 7B batch-8 cached step 6.78 ->
// 6.66 ms, prefix-mode step at 256 rows 6.96 -> 6.91 ms.  (The large-tile epilogue measured
// slower that way: 8B refresh 30.1 -> 31.1 ms, so it keeps plain stores.)
constexpr int MD_BN = 128, MD_DK = 64, MD_NSTG = 3, MD_THREADS = 512;
constexpr int MD_A = kMidRows * MD_DK * 2;  // A (activation) bytes per stage
constexpr int MD_STG = MD_A + MD_BN * MD_DK * 2;
constexpr int MD_SMEM = MD_NSTG * MD_STG;   // 144 KB
constexpr int MD_TL = 132;                  // row stride (floats) of the epilogue tile
static_assert(kMidRows * MD_TL * 4 <= MD_SMEM, "epilogue tile fits in the operand ring");
static_assert(BG_T == kBigTile, "large tile edge");

// Epilogue of a whole tile in LDS (rows 0..255, tile-local virtual columns 0..127 at
// vc0) in wrow_s2's virtual order.  Only STORE, F32 and SWIGLU tiles are whole.
template <int EPI>
__device__ void mid_epilogue(const float* tile, int M, int vc0, int Nv, const EpiArgs& e) {
  if constexpr (EPI == EPI_SWIGLU) {
    // 64 outputs per row: column c of the tile's span takes gate 64(c/32) + c%32, up +32;
    // 4 adjacent outputs per thread
    uint16_t* y = (uint16_t*)e.y;
    const bool vec = e.F % 4 == 0 && aligned_to(y, 8);
    for (int i = threadIdx.x; i < kMidRows * 16; i += blockDim.x) {
      const int m = i >> 4, c = 4 * (i & 15);
      const int vg = 64 * (c >> 5) + (c & 31);
      if (m >= M || vc0 + vg >= Nv) continue;
      const float4 gt = *reinterpret_cast<const float4*>(tile + m * MD_TL + vg);
      const float4 up = *reinterpret_cast<const float4*>(tile + m * MD_TL + vg + 32);
      uint16_t* p = y + (int64_t)m * e.F + vc0 / 2 + c;
      if (vec && vc0 + vg + 3 < Nv) {
        st_dev(p, u16x4{swiglu_bf16(gt.x, up.x), swiglu_bf16(gt.y, up.y),
                        swiglu_bf16(gt.z, up.z), swiglu_bf16(gt.w, up.w)});
      } else {
        const float gg[4] = {gt.x, gt.y, gt.z, gt.w}, uu[4] = {up.x, up.y, up.z, up.w};
        for (int u = 0; u < 4 && vc0 + vg + u < Nv; ++u) p[u] = swiglu_bf16(gg[u], uu[u]);
      }
    }
  } else if constexpr (EPI == EPI_STORE || EPI == EPI_F32) {
    epilogue<uint16_t, EPI>(tile, MD_TL, kMidRows, 0, vc0, M, Nv, e);
  }
  // residual and QKV GEMMs are always split (the plan gives them no whole tiles)
}

template <int MAP, int EPI, bool FULL>
__global__ __launch_bounds__(MD_THREADS, 1) void gemm_mid_bf16(
    const uint16_t* __restrict__ X, int ldx, const uint16_t* __restrict__ W, int M, int Nv, int K,
    int ndp, int splits, int kst, int nunits, float* __restrict__ part, EpiArgs e) {
  extern __shared__ __attribute__((aligned(16))) unsigned char md_smem[];
  const int tid = threadIdx.x;
  const int w = tid >> 6, wm = w & 3, wn = w >> 2, l = tid & 63, lr = l & 31, g = l >> 5;
  const int Nt = Nv - ndp * MD_BN;  // row stride of the partials
  // 16-byte chunk c of tile row r sits in slot c ^ ((r >> 1) & 7) of the row's 128 bytes.
  // LDS serves a 16-byte-per-lane read 16 lanes per clock from 64 four-byte banks (256
  // bytes); an operand read puts 16 consecutive rows at one k offset in those lanes.  Rows
  // r and r + 1 already fall in different halves of the 256 bytes, so the key changes
  // every second row and the 16 rows land in 16 distinct 16-byte slots (keyed by r & 7,
  // rows r and r + 8 collided: half the read rate, measured).  For 64-byte rows (four
  // per 256 bytes) the key is (r >> 2) & 3.
  auto swz = [](int r) { return (r >> 1) & 7; };

  for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
    const bool whole = u < ndp;
    int tile = u, split = 0, kb = 0, ke = K;
    if (!whole) {
      const int v = u - ndp;
      tile = ndp + v / splits;
      split = v % splits;
      kb = split * kst * MD_DK;
      ke = min(K, kb + kst * MD_DK);
    }
    const int vc0 = tile * MD_BN;
    const int nst = (ke - kb) / MD_DK;

    // wave w fills A rows 32w .. +32 and B rows 16w .. +16, 8 rows per load instruction
    // (lane l: row + l/8, chunk slot l%8); rows past M / columns past Nv read a clamped
    // valid row whose results are never stored
    const uint16_t* asrc[4];
    const uint16_t* bsrc[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 32 * w + 8 * i + (l >> 3);
      asrc[i] = X + (int64_t)min(row, M - 1) * ldx + kb + ((l & 7) ^ swz(row)) * 8;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 16 * w + 8 * i + (l >> 3);
      bsrc[i] = W + (int64_t)wrow_s2<MAP>(min(vc0 + row, Nv - 1), e.F) * K + kb +
                ((l & 7) ^ swz(row)) * 8;
    }
    // Below 256 rows (FULL false), rows past M are neither loaded nor multiplied: wave
    // w's activation loads cover rows 32w + 8i for i < nxi, and a wave whose 64-row band
    // starts at or past M skips its MFMAs (bit-identical; 96 rows x 24576 x 4096: 80.3 ->
    // 62.5 us, prefix workload 976 -> 956 ms per generation).  Rows past M that a band
    // still covers read stale LDS rows; their results are never stored.  At 256 rows the
    // FULL instantiation has no such branches (they cost the 7B batch-8 step 1.4 %).
    const int nxi =
        FULL ? 4 : __builtin_amdgcn_readfirstlane(min(4, max(0, (M - 32 * w + 7) / 8)));
    const bool act = FULL || 64 * wm < M;
    auto issue = [&](int st) {
      unsigned char* base = md_smem + (st % MD_NSTG) * MD_STG;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nxi) __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(asrc[i] + st * MD_DK),
            (__attribute__((address_space(3))) void*)(base + (32 * w + 8 * i) * (MD_DK * 2)), 16,
            0, 0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(bsrc[i] + st * MD_DK),
            (__attribute__((address_space(3))) void*)(base + MD_A + (16 * w + 8 * i) * (MD_DK * 2)),
            16, 0, 0);
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    auto frag = [&](int slot, int kk, u32x4* a, u32x4* b) {
      const unsigned char* base = md_smem + slot * MD_STG;
      const int c = 2 * kk + g;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + lr;
        a[i] = *reinterpret_cast<const u32x4*>(base + r * (MD_DK * 2) + ((c ^ swz(r)) * 16));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 64 * wn + 32 * j + lr;
        b[j] = *reinterpret_cast<const u32x4*>(base + MD_A + r * (MD_DK * 2) + ((c ^ swz(r)) * 16));
      }
    };
    auto compute = [&](int slot) {
      u32x4 a[2][2], b[2][2];
      frag(slot, 0, a[0], b[0]);
#pragma unroll
      for (int kk = 0; kk < MD_DK / 16; ++kk) {
        if (kk + 1 < MD_DK / 16) frag(slot, kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = mfma32(as_bf16x8(a[kk & 1][i]), as_bf16x8(b[kk & 1][j]), acc[i][j]);
      }
      // issue order: the four operand reads of step 0, then the next step's reads
      // alternating with this step's MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 0x100: LDS reads
#pragma unroll
      for (int kk = 0; kk < MD_DK / 16 - 1; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 0x008: MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };
    // s_waitcnt with only vmcnt = n (expcnt and lgkmcnt left at their maximum)
#define DLLM_VMWAIT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
    for (int st = 0; st < MD_NSTG - 1 && st < nst; ++st) issue(st);
    for (int st = 0; st < nst; ++st) {
      // this wave's loads of stage st have landed once at most its nxi + 2 loads of
      // stage st + 1 are still in flight; the barrier then covers every wave's, and every
      // wave is done with the slot that stage st + 2 refills
      if (st + 1 < nst) {
        if (nxi == 4) DLLM_VMWAIT(6);
        else if (nxi == 3) DLLM_VMWAIT(5);
        else if (nxi == 2) DLLM_VMWAIT(4);
        else if (nxi == 1) DLLM_VMWAIT(3);
        else DLLM_VMWAIT(2);
      } else {
        DLLM_VMWAIT(0);
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (st + MD_NSTG - 1 < nst) issue(st + MD_NSTG - 1);
      if (act) compute(st % MD_NSTG);
    }
#undef DLLM_VMWAIT
    __syncthreads();  // the operand ring is free: the epilogue tile and the next unit reuse it

    // accumulator (i, j, v): tile row 64 wm + 32 i + acc_row(v, g), column 64 wn + 32 j + lr
    if (whole) {
      float* t = reinterpret_cast<float*>(md_smem);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            t[(64 * wm + 32 * i + acc_row(v, g)) * MD_TL + 64 * wn + 32 * j + lr] = acc[i][j][v];
      __syncthreads();
      mid_epilogue<EPI>(t, M, vc0, Nv, e);
      __syncthreads();
    } else {
      float* pp = part + (int64_t)split * M * Nt;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int vc = vc0 + 64 * wn + 32 * j + lr;
        if (vc >= Nv) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = 64 * wm + 32 * i + acc_row(v, g);
            if (r < M) st_dev(&pp[(int64_t)r * Nt + (vc - ndp * MD_BN)], acc[i][j][v]);
          }
      }
    }
  }
}

// ============================================================================
// fp32 SIMT GEMM (fp32 models): 32x128 tiles, K % 16 == 0
// ============================================================================
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32(const float* __restrict__ X, int ldx,
                                                const float* __restrict__ W, int M, int Nv, int K,
                                                EpiArgs e) {
  constexpr int BK = 16;
  __shared__ float Xs[BK][33];
  __shared__ float Ws[BK][129];
  __shared__ float tile[32 * TL];
  const int tn = blockIdx.x, tm = blockIdx.y;
  const int m0 = tm * 32, vc0 = tn * 128;
  const int tid = threadIdx.x, tr = tid >> 5, tc = tid & 31;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int i = 0; i < 2; ++i) {
      int ee = tid + 256 * i;
      int r = ee >> 4, kk = ee & 15;
      Xs[kk][r] = (m0 + r < M) ? X[(int64_t)(m0 + r) * ldx + k0 + kk] : 0.f;
    }
    for (int i = 0; i < 8; ++i) {
      int ee = tid + 256 * i;
      int r = ee >> 4, kk = ee & 15;
      int vc = vc0 + r;
      Ws[kk][r] = (vc < Nv) ? W[(int64_t)wrow_of<EPI>(vc, e.F) * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = Xs[kk][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Ws[kk][tc + 32 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) tile[(tr * 4 + i) * TL + tc + 32 * j] = acc[i][j];
  __syncthreads();
  epilogue<float, EPI>(tile, TL, 32, m0, vc0, M, Nv, e);
}


// ============================================================================
// split-K reduction + epilogue for the skinny GEMM (partials in 64-column virtual order)
// ============================================================================
// One thread per 4 consecutive outputs (helpers in kernels.h).

// One RoPE pair of the QKV epilogue (head_dim 128): head slot hs (q heads, then k, then
// v), dims d and d + 64 of row m, with the sums x1 and x2.  q and k are rotated at the
// row's position; v is written to the transposed cache.
__device__ __forceinline__ void qkv_pair(const EpiArgs& e, int m, int hs, int d, float x1,
                                         float x2) {
  const int bs = m / e.R, ri = m % e.R, pos = e.pos0 + ri;
  if (hs < e.Hq + e.Hkv) {
    uint16_t* dst = (hs < e.Hq)
        ? (uint16_t*)e.qo + (((int64_t)bs * e.Hq + hs) * e.R + ri) * 128
        : (uint16_t*)e.kc + (((int64_t)bs * e.Hkv + (hs - e.Hq)) * e.Sp + pos) * 128;
    const float cs = e.rcos[(int64_t)pos * 64 + d], sn = e.rsin[(int64_t)pos * 64 + d];
    dst[d] = f2bf(x1 * cs - x2 * sn);
    dst[d + 64] = f2bf(x2 * cs + x1 * sn);
  } else {
    uint16_t* dst = (uint16_t*)e.vtc + ((int64_t)bs * e.Hkv + (hs - e.Hq - e.Hkv)) * 128 * (int64_t)e.Sp;
    dst[vt_off(d, pos, 128)] = f2bf(x1);
    dst[vt_off(d + 64, pos, 128)] = f2bf(x2);
  }
}

// Split-K reduction + epilogue over the partial columns [0, pv.N), i.e. the virtual
// output columns [pv.vbase, pv.vbase + pv.N), in the producing GEMM's virtual order
// (pv.order): the 64-column order of wrow_s2 (SwiGLU: 32 gate columns then the matching
// 32 up columns; QKV: one head slot per 128 columns, dims 0..31, 64..95, 32..63,
// 96..127) or the large tiles' 128-column order of wrow_of (64 + 64; dims in order).
// QKV: workgroups [0, qk_blocks) take the q and k head slots (the first nqk slots of
// the span), one thread per (row, slot, 4 rotated pairs); the rest take 32 rows x 32
// dims of one V head slot each, transposed through LDS so that the stores into the
// blocked Vt cache (keys contiguous) are 32 consecutive keys per dim instead of one
// 2-byte store per key.
template <int EPI>
__global__ __launch_bounds__(256) void reduce_epilogue(PartView pv, EpiArgs e, int nqk,
                                                       int qk_blocks) {
  const int M = pv.M, Nt = pv.N;
  const int64_t i4 = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) * 4;
  if constexpr (EPI == EPI_STORE || EPI == EPI_F32) {
    // Nt % 4 == 0: 4 outputs of one row
    if (i4 >= (int64_t)M * Nt) return;
    const int m = (int)(i4 / Nt), c = (int)(i4 % Nt), vc = pv.vbase + c;
    const float4 v = scale4(sum_split4(pv, m, c), row_rms_factor(e, m));
    if constexpr (EPI == EPI_F32) {
      float4 o = make_float4(v.x * e.scale, v.y * e.scale, v.z * e.scale, v.w * e.scale);
      *reinterpret_cast<float4*>((float*)e.y + (int64_t)m * e.ldy + vc) = o;
    } else {
      uint16_t* y = (uint16_t*)e.y + (int64_t)m * e.ldy + vc;
      y[0] = f2bf(v.x); y[1] = f2bf(v.y); y[2] = f2bf(v.z); y[3] = f2bf(v.w);
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // output column c of the span: gate at partial column 64(c/32) + c%32, up 32 further
    // (128-column order: 128(c/64) + c%64, up 64 further)
    const int nout = Nt / 2;
    if (i4 >= (int64_t)M * nout) return;
    const int m = (int)(i4 / nout), c = (int)(i4 % nout);
    const int gw = pv.order ? 64 : 32;
    const int vg = 2 * gw * (c / gw) + (c % gw);
    const float r = row_rms_factor(e, m);
    const float4 gt = scale4(sum_split4(pv, m, vg), r);
    const float4 up = scale4(sum_split4(pv, m, vg + gw), r);
    uint16_t* y = (uint16_t*)e.y + (int64_t)m * e.F + pv.vbase / 2 + c;
    // written through like the GEMM partials (d_ffn % 64 == 0 keeps y 8-byte aligned)
    st_dev(y, u16x4{swiglu_bf16(gt.x, up.x), swiglu_bf16(gt.y, up.y), swiglu_bf16(gt.z, up.z),
                    swiglu_bf16(gt.w, up.w)});
  } else if constexpr (EPI == EPI_QKV) {
    if ((int)blockIdx.x >= qk_blocks) {  // V: uniform per workgroup
      __shared__ float tile[32][33];     // [row][dim]; odd stride: conflict-free columns
      const int nv = Nt / 128 - nqk;
      const int vb = (int)blockIdx.x - qk_blocks;
      const int hl = nqk + (vb >> 2) % nv, m0 = ((vb >> 2) / nv) * 32, q = vb & 3;
      // virtual columns [32q, 32q + 32) of the slot hold one run of 32 dims: the 64-column
      // order keeps dims 0-31, 64-95, 32-63, 96-127; the 128-column order keeps them in place
      const int dbase = pv.order ? 32 * q : (q & 1) * 64 + (q >> 1) * 32;
      const int t = threadIdx.x;
      {
        const int mr = t >> 3, m = m0 + mr, j = 4 * (t & 7);
        if (m < M) {
          const float4 v = scale4(sum_split4(pv, m, 128 * hl + 32 * q + j), row_rms_factor(e, m));
          tile[mr][j] = v.x; tile[mr][j + 1] = v.y; tile[mr][j + 2] = v.z; tile[mr][j + 3] = v.w;
        }
      }
      __syncthreads();
      const int mr = t & 31, m = m0 + mr, d0 = (t >> 5) * 4;
      if (m < M) {
        const int bs = m / e.R, ri = m % e.R, pos = e.pos0 + ri;
        const int hs = pv.vbase / 128 + hl;
        uint16_t* dst = (uint16_t*)e.vtc +
                        ((int64_t)bs * e.Hkv + (hs - e.Hq - e.Hkv)) * 128 * (int64_t)e.Sp;
#pragma unroll
        // written through: the attention kernel that follows reads the cache from every XCD
        for (int i = 0; i < 4; ++i) st_dev(&dst[vt_off(dbase + d0 + i, pos, 128)], f2bf(tile[mr][d0 + i]));
      }
      return;
    }
    // (row m, head slot hs, dims d..d+3 < 64) -> pairs (d, d+64); head_dim 128
    const int nslot = nqk;
    if (i4 >= (int64_t)M * nslot * 64) return;
    const int m = (int)(i4 / (nslot * 64));
    const int rem = (int)(i4 % (nslot * 64));
    const int hl = rem / 64, d = rem % 64;
    // the pair (d, d + 64) of head slot hl: 64-column order keeps dims 0-31, 64-95,
    // 32-63, 96-127; 128-column order keeps them in place
    const int c = pv.order ? 128 * hl + d : 64 * (2 * hl + (d >> 5)) + (d & 31);
    const int cb = pv.order ? c + 64 : c + 32;
    const float r = row_rms_factor(e, m);
    const float4 a = scale4(sum_split4(pv, m, c), r);
    const float4 b = scale4(sum_split4(pv, m, cb), r);
    const int hs = pv.vbase / 128 + hl;
    if (hs < e.Hq + e.Hkv) {
      // q or k: the four rotated pairs as two 8-byte stores (dims d..d+3, d+64..d+67)
      const int bs = m / e.R, ri = m % e.R, pos = e.pos0 + ri;
      uint16_t* dst = (hs < e.Hq)
          ? (uint16_t*)e.qo + (((int64_t)bs * e.Hq + hs) * e.R + ri) * 128
          : (uint16_t*)e.kc + (((int64_t)bs * e.Hkv + (hs - e.Hq)) * e.Sp + pos) * 128;
      const float4 cs = *reinterpret_cast<const float4*>(e.rcos + (int64_t)pos * 64 + d);
      const float4 sn = *reinterpret_cast<const float4*>(e.rsin + (int64_t)pos * 64 + d);
      // written through (device-coherent stores): 4.185 -> 4.181 ms per 8B cached step
      st_dev(dst + d, u16x4{f2bf(a.x * cs.x - b.x * sn.x), f2bf(a.y * cs.y - b.y * sn.y),
                            f2bf(a.z * cs.z - b.z * sn.z), f2bf(a.w * cs.w - b.w * sn.w)});
      st_dev(dst + d + 64, u16x4{f2bf(b.x * cs.x + a.x * sn.x), f2bf(b.y * cs.y + a.y * sn.y),
                                 f2bf(b.z * cs.z + a.z * sn.z), f2bf(b.w * cs.w + a.w * sn.w)});
    } else {
      qkv_pair(e, m, hs, d + 0, a.x, b.x);
      qkv_pair(e, m, hs, d + 1, a.y, b.y);
      qkv_pair(e, m, hs, d + 2, a.z, b.z);
      qkv_pair(e, m, hs, d + 3, a.w, b.w);
    }
  }
}

hipError_t launch_reduce_epilogue(int epi, const PartView& pv, const EpiArgs& e, hipStream_t st) {
  int64_t n4 = 0;
  int nqk = 0, qkb = 0, vblocks = 0;
  if (epi == EPI_STORE || epi == EPI_F32) n4 = (int64_t)pv.M * pv.N / 4;
  else if (epi == EPI_SWIGLU) n4 = (int64_t)pv.M * (pv.N / 2) / 4;
  else if (epi == EPI_QKV) {
    // the span's slots are q and k heads up to slot Hq + Hkv, V heads after it
    const int nslot = pv.N / 128;
    nqk = std::max(0, std::min(nslot, e.Hq + e.Hkv - pv.vbase / 128));
    n4 = (int64_t)pv.M * nqk * 16;
    qkb = (int)((n4 + 255) / 256);
    vblocks = (nslot - nqk) * ((pv.M + 31) / 32) * 4;
  } else return hipErrorInvalidValue;
  const int64_t blocks64 = (n4 + 255) / 256 + vblocks;
  if (blocks64 <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)blocks64;
  switch (epi) {
    case EPI_STORE: reduce_epilogue<EPI_STORE><<<blocks, 256, 0, st>>>(pv, e, 0, 0); break;
    case EPI_F32: reduce_epilogue<EPI_F32><<<blocks, 256, 0, st>>>(pv, e, 0, 0); break;
    case EPI_SWIGLU: reduce_epilogue<EPI_SWIGLU><<<blocks, 256, 0, st>>>(pv, e, 0, 0); break;
    case EPI_QKV: reduce_epilogue<EPI_QKV><<<blocks, 256, 0, st>>>(pv, e, nqk, qkb); break;
  }
  return hipGetLastError();
}

// ============================================================================
// planning and dispatch
// ============================================================================
// compute units of the current device (256 on MI355X; 256 when no device is visible)
static int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0)
      n = cus;
    else
      n = 256;
  }
  return n;
}

GemmPlan gemm_plan(int dtype, int M, int Nv, int K, int epi) {
  GemmPlan p;
  if (dtype == F32) {
    p.kind = GEMM_F32;
    p.ntn = (Nv + 127) / 128;
    p.ntm = (M + 31) / 32;
    p.kchunk = K;
    return p;
  }
  if (M <= kSkinnyRows) {
    p.kind = GEMM_SKINNY;
    p.mt = (M <= 16) ? 1 : (M <= 32) ? 2 : 4;
    p.ntn = (Nv + 15) / 16;  // 16-column groups
    p.ntm = 1;
    // per-wave K sub-range KS (the workgroup covers 8 KS): among 256/192/128/64 with
    // K % (8 KS) == 0 whose activation slice fits the LDS (M > 32 rows: KS <= 128), those
    // that give every workgroup at least 4 of the 16-column groups to walk (a workgroup
    // with fewer spends most of its time staging its activation slice and waiting for its
    // first weights: the 8B output projection, 2 groups per workgroup at 256, runs
    // 10.3 us at 256 and 8.4 us at 128) compete on one workgroup's critical path: the
    // most groups g it walks, plus its activation slice (as many bytes as MT groups'
    // weights), times KS, plus 16 MT per group (a group's fixed cost: the cross-wave sum
    // and partial stores of its MT x 16 rows); larger KS on ties; else the largest (32
    // if none).  On the 8B cached step (same process, alternating rounds) this picks
    // what measured fastest: the down projection (K = 12288, 256 groups) takes 192,
    // 8 K ranges of 32 workgroups walking 8 groups each, where 256 gives 6 ranges of 42
    // of which 4 walk 7 groups and the rest 6 (4.168 -> 4.109 ms); QKV takes 128, 12
    // groups behind a 64 KB slice instead of 6 behind 128 KB (4.147 -> 4.121 ms);
    // gate/up stays at 256 (128: 4.178 ms), the output projection at 128 (64: 4.185
    // ms), the LM head at 256 (128 measured the same).  At 64 rows (prefix-mode steps)
    // the output projection stays at 128 too (64: 935 -> 940 ms per prefix-workload
    // generation).
    int ks = 32;
    bool found = false;
    long best = -1;
    const int ngrp16 = (Nv + 15) / 16;
    for (int c : {256, 192, 128, 64}) {
      if (K % (8 * c) != 0 || (p.mt > 2 && c > 128)) continue;
      const int per_range = std::max(1, num_cus() / (K / (8 * c)));  // workgroups per K range
      if (!found) { ks = c; found = true; }
      if (ngrp16 >= 4 * per_range) {
        const int wgs = std::min(per_range, ngrp16);
        const long g = (ngrp16 + wgs - 1) / wgs;
        const long cost = (g + p.mt) * c + 16L * p.mt * g;
        if (best < 0 || cost < best) { best = cost; ks = c; }
      }
    }
    p.kchunk = 8 * ks;
    p.splits = K / p.kchunk;
    p.part_floats = (size_t)p.splits * ((Nv + 15) / 16) * (p.mt * 16 * 16);  // blocked layout
    p.deferred = true;  // partials reduced by the next RMSNorm or by reduce_epilogue
    p.reduce = (epi != EPI_RESID);
    return p;
  }
  if (M <= kMidRows && K % MD_DK == 0) {
    // one 256-row tile: residual and QKV GEMMs split every tile over K into about one
    // unit per CU; the others run whole tiles and split only a ragged last round
    p.kind = GEMM_MID;
    const int P = num_cus();
    const int tiles = (Nv + MD_BN - 1) / MD_BN;
    const int ns = K / MD_DK;
    int S = 1, ndp = 0;
    if (epi == EPI_RESID || epi == EPI_QKV) {
      S = P / tiles;
    } else {
      const int tail = tiles % P;
      // the reduction of a split tail reads float4 columns
      S = (tail > 0 && Nv % 4 == 0) ? P / tail : 1;
      ndp = (S <= 1) ? tiles : tiles - tail;
    }
    S = std::max(1, std::min(S, ns));
    const int kst = (ns + S - 1) / S;  // stages per split; no split is empty
    S = (ns + kst - 1) / kst;
    p.ntn = tiles;
    p.ntm = 1;
    p.splits = S;
    p.kchunk = kst * MD_DK;
    p.ndp = ndp;
    p.units = ndp + (tiles - ndp) * S;
    if (ndp < tiles) {
      p.part_floats = (size_t)S * M * (Nv - ndp * MD_BN);
      p.deferred = true;
      p.reduce = (epi != EPI_RESID);
    }
    return p;
  }
  // large GEMMs: 256x256 tiles unless their count fills the chip much worse than the
  // 128x128 tiles' (the large tile does ~15% more work per unit time)
  auto fill = [](int tiles, int slots) {
    const int waves = (tiles + slots - 1) / slots;
    return (double)tiles / ((double)waves * slots);
  };
  const int big_tiles = ((Nv + BG_T - 1) / BG_T) * ((M + BG_T - 1) / BG_T);
  const int small_tiles = ((Nv + 127) / 128) * ((M + 127) / 128);
  const bool big_fills = (epi == EPI_RESID && big_tiles < 256) ||
                         1.15 * fill(big_tiles, 256) >= fill(small_tiles, 512);
  // 256 <= M < 512 (one row tile of 256): the large tile reads each weight tile once,
  // while the 128-row tiles read it twice; worth it once it fills a round of CUs
  const bool big_mid = M >= 256 && M < 512 && big_tiles >= 256;
  // Non-residual GEMMs whose ragged last round of large tiles is made of whole column
  // tiles: the leading columns run as whole tiles, and the trailing ones either split over
  // K into about one round of large-tile pieces (partials, reduce_epilogue; e.g. the
  // 2024-row QKV: 256 large tiles, then 2 x 128 pieces), or, where a round holds fewer
  // than two pieces per tail tile, as 128x128 tiles when those fill a round of CUs.  (The
  // 2024-row QKV took 30.19 ms per 8B refresh with its tail as 512 small tiles, 29.98 ms
  // split over K.)
  if (K % TB_K == 0 && M >= 512 && epi != EPI_RESID) {
    const int P = num_cus();
    const int ntn = (Nv + BG_T - 1) / BG_T, ntm = (M + BG_T - 1) / BG_T;
    const int tail = (ntn * ntm) % P;
    const int S = tail ? std::min(P / tail, K / TB_K) : 0;
    // the reduction reads float4 columns and, for QKV, whole head slots
    if (ntn * ntm > P && tail % ntm == 0 && S >= 2 && Nv % 4 == 0 &&
        (epi != EPI_QKV || Nv % 128 == 0)) {
      p.kind = GEMM_BIG;
      p.ntn = ntn;
      p.ntm = ntm;
      p.ndp = ntn - tail / ntm;
      const int per = (K + S - 1) / S;
      p.kchunk = (per + TB_K - 1) / TB_K * TB_K;
      p.splits = (K + p.kchunk - 1) / p.kchunk;
      p.part_floats = (size_t)p.splits * M * (Nv - p.ndp * BG_T);
      p.deferred = true;
      p.reduce = true;
      return p;
    }
    if (ntn * ntm > P && tail % ntm == 0 && 4 * tail >= P) {
      // the tail's columns as 128x128 tiles (4 per large tile) fill a round of CUs: run
      // them on the tiled kernel, whole K, epilogue in place (no partials)
      p.kind = GEMM_BIG;
      p.ntn = ntn;
      p.ntm = ntm;
      p.ndp = ntn - tail / ntm;
      p.tail_tiled = true;
      p.kchunk = K;
      p.splits = 1;
      return p;
    }
  }
  if (K % TB_K == 0 && ((M >= 512 && big_fills) || big_mid)) {
    p.kind = GEMM_BIG;
    p.ntn = (Nv + BG_T - 1) / BG_T;
    p.ntm = (M + BG_T - 1) / BG_T;
    const int tiles = p.ntn * p.ntm;
    int splits = 1;
    if (epi == EPI_RESID && tiles < 256) {  // fill the chip: split K, deferred partials
      splits = (256 + tiles - 1) / tiles;
      if (splits > K / TB_K) splits = K / TB_K;
    }
    const int per = (K + splits - 1) / splits;
    p.kchunk = (per + TB_K - 1) / TB_K * TB_K;
    p.splits = (K + p.kchunk - 1) / p.kchunk;
    if (p.splits > 1) {
      p.part_floats = (size_t)p.splits * M * Nv;
      p.deferred = true;
    }
    return p;
  }
  p.kind = GEMM_TILED;
  p.ntn = (Nv + 127) / 128;
  p.ntm = (M + 127) / 128;
  const int ks = TB_K, target = 512;
  const int tiles = p.ntn * p.ntm;
  int splits = 1;
  // Residual partials are plain stores folded by the next norm; the other epilogues hand
  // split partials over through coherent stores and an arrival counter, which costs more
  // than the extra parallelism gains unless the tile count is small (measured at
  // M = 256: 72 tiles of a 4608-wide QKV take 61 us unsplit, 74-88 us with 2-8 splits).
  if (tiles < target && (epi == EPI_RESID || tiles < 64)) {
    splits = (target + tiles - 1) / tiles;
    int maxs = K / ks;
    if (splits > maxs) splits = maxs;
    if (splits > 32) splits = 32;
    if (splits < 1) splits = 1;
  }
  int per = (K + splits - 1) / splits;
  p.kchunk = (per + ks - 1) / ks * ks;
  p.splits = (K + p.kchunk - 1) / p.kchunk;
  if (p.splits > 1) {
    p.part_floats = (size_t)p.splits * M * Nv;
    p.deferred = (epi == EPI_RESID);
    p.counters = p.deferred ? 0 : tiles;
  }
  return p;
}

template <int EPI>
static hipError_t launch_epi(int dtype, const GemmPlan& p, const void* X, int ldx, const void* W,
                             int M, int Nv, int K, const EpiArgs& e, float* part, int* counters,
                             hipStream_t st) {
  if (p.kind == GEMM_F32) {
    gemm_f32<EPI><<<dim3(p.ntn, p.ntm), 256, 0, st>>>((const float*)X, ldx, (const float*)W, M,
                                                     Nv, K, e);
  } else if (p.kind == GEMM_SKINNY) {
    // persistent: one 8-wave workgroup per CU, a whole number of workgroups per K range
    const int ngrp = (Nv + 15) / 16;
    int per_split = num_cus() / p.splits;
    if (per_split < 1) per_split = 1;
    if (per_split > ngrp) per_split = ngrp;
    dim3 grid(per_split * p.splits);
    const uint16_t* Xb = (const uint16_t*)X;
    const uint16_t* Wb = (const uint16_t*)W;
    constexpr int MAP = (EPI == EPI_SWIGLU || EPI == EPI_QKV) ? EPI : EPI_STORE;
#define DLLM_SKINNY(MTV, KSV)                                                           \
    gemm_skinny_bf16<MAP, MTV, KSV><<<grid, 512, 0, st>>>(Xb, ldx, Wb, M, Nv, K, e.F,  \
                                                         p.splits, ngrp, part)
    const int ks = p.kchunk / 8;
    if (p.mt == 1) {
      if (ks == 256) DLLM_SKINNY(1, 256);
      else if (ks == 192) DLLM_SKINNY(1, 192);
      else if (ks == 128) DLLM_SKINNY(1, 128);
      else if (ks == 64) DLLM_SKINNY(1, 64);
      else DLLM_SKINNY(1, 32);
    } else if (p.mt == 2) {
      if (ks == 256) DLLM_SKINNY(2, 256);
      else if (ks == 192) DLLM_SKINNY(2, 192);
      else if (ks == 128) DLLM_SKINNY(2, 128);
      else if (ks == 64) DLLM_SKINNY(2, 64);
      else DLLM_SKINNY(2, 32);
    } else {
      if (ks == 128) DLLM_SKINNY(4, 128);
      else if (ks == 64) DLLM_SKINNY(4, 64);
      else DLLM_SKINNY(4, 32);
    }
#undef DLLM_SKINNY
  } else if (p.kind == GEMM_MID) {
    constexpr int MAP = (EPI == EPI_SWIGLU || EPI == EPI_QKV) ? EPI : EPI_STORE;
    static bool mid_attr_set = false;  // opt in to more than 64 KB of dynamic LDS once
    if (!mid_attr_set) {
      for (const void* f : {reinterpret_cast<const void*>(&gemm_mid_bf16<MAP, EPI, true>),
                            reinterpret_cast<const void*>(&gemm_mid_bf16<MAP, EPI, false>)}) {
        hipError_t err =
            hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, MD_SMEM);
        if (err != hipSuccess) return err;
      }
      mid_attr_set = true;
    }
    const int grid = std::min(p.units, num_cus());
    if (M >= kMidRows)
      gemm_mid_bf16<MAP, EPI, true><<<grid, MD_THREADS, MD_SMEM, st>>>(
          (const uint16_t*)X, ldx, (const uint16_t*)W, M, Nv, K, p.ndp, p.splits,
          p.kchunk / MD_DK, p.units, part, e);
    else
      gemm_mid_bf16<MAP, EPI, false><<<grid, MD_THREADS, MD_SMEM, st>>>(
          (const uint16_t*)X, ldx, (const uint16_t*)W, M, Nv, K, p.ndp, p.splits,
          p.kchunk / MD_DK, p.units, part, e);
  } else if (p.kind == GEMM_BIG) {
    static bool attr_set = false;  // opt in to more than 64 KB of dynamic LDS once
    if (!attr_set) {
      hipError_t err = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&gemm_big_bf16<EPI, BG_DK, BG_NSTG>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, BG_SMEM);
      if (err != hipSuccess) return err;
      attr_set = true;
    }
    if (p.ndp > 0) {  // whole column tiles [0, ndp), then the split tail
      gemm_big_bf16<EPI, BG_DK, BG_NSTG><<<dim3(p.ndp, p.ntm, 1), BG_THREADS, BG_SMEM, st>>>(
          (const uint16_t*)X, ldx, (const uint16_t*)W, M, Nv, K, K, 1, part, e, 0, 0);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      if (p.tail_tiled) {
        const int tn0 = p.ndp * (BG_T / 128);
        gemm_tiled_bf16<EPI><<<dim3((M + 127) / 128, (Nv + 127) / 128 - tn0, 1), 256, 0, st>>>(
            (const uint16_t*)X, ldx, (const uint16_t*)W, M, Nv, K, K, 1, part, counters, e, tn0);
        return hipGetLastError();
      }
      gemm_big_bf16<EPI, BG_DK, BG_NSTG>
          <<<dim3(p.ntn - p.ndp, p.ntm, p.splits), BG_THREADS, BG_SMEM, st>>>(
              (const uint16_t*)X, ldx, (const uint16_t*)W, M, Nv, K, p.kchunk, p.splits, part, e,
              p.ndp, p.ndp * BG_T);
    } else {
      gemm_big_bf16<EPI, BG_DK, BG_NSTG><<<dim3(p.ntn, p.ntm, p.splits), BG_THREADS, BG_SMEM, st>>>(
          (const uint16_t*)X, ldx, (const uint16_t*)W, M, Nv, K, p.kchunk, p.splits, part, e, 0, 0);
    }
  } else {
    gemm_tiled_bf16<EPI><<<dim3(p.ntm, p.ntn, p.splits), 256, 0, st>>>(
        (const uint16_t*)X, ldx, (const uint16_t*)W, M, Nv, K, p.kchunk, p.splits, part, counters,
        e, 0);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epi, const GemmPlan& p, const void* X, int ldx,
                       const void* W, int M, int Nv, int K, const EpiArgs& e, float* part,
                       int* counters, hipStream_t st) {
  if (M <= 0 || Nv <= 0) return hipSuccess;
  hipError_t err = launch_gemm_only(dtype, epi, p, X, ldx, W, M, Nv, K, e, part, counters, st);
  if (err != hipSuccess) return err;
  if (p.reduce) return launch_reduce_epilogue(epi, p.view(part, M, Nv), e, st);
  return hipSuccess;
}

hipError_t launch_gemm_only(int dtype, int epi, const GemmPlan& p, const void* X, int ldx,
                            const void* W, int M, int Nv, int K, const EpiArgs& e, float* part,
                            int* counters, hipStream_t st) {
  switch (epi) {
    case EPI_STORE: return launch_epi<EPI_STORE>(dtype, p, X, ldx, W, M, Nv, K, e, part, counters, st);
    case EPI_F32: return launch_epi<EPI_F32>(dtype, p, X, ldx, W, M, Nv, K, e, part, counters, st);
    case EPI_RESID: return launch_epi<EPI_RESID>(dtype, p, X, ldx, W, M, Nv, K, e, part, counters, st);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(dtype, p, X, ldx, W, M, Nv, K, e, part, counters, st);
    case EPI_QKV: return launch_epi<EPI_QKV>(dtype, p, X, ldx, W, M, Nv, K, e, part, counters, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dllm
