// Dense projections y = x . W^T of the transformer (QKV, output, gate/up, down, LM head)
// with their element-wise tails fused into the epilogue.
//
// Every kernel produces an fp32 tile of 128 "virtual" output columns in LDS and hands it
// to one epilogue (kernels.h: EpiKind):
//   QKV    : RoPE on q and k (rotate-half, pairs j and j + D/2, table cos/sin[pos][j]),
//            q scattered to [B][Hq][R][D], k into the cache K [B][Hkv][Sp][D], v into the
//            transposed cache Vt [B][Hkv][D][Sp] (the block's own K/V written in place);
//   SWIGLU : a virtual tile is 64 gate rows + the matching 64 up rows of W, so the tile
//            holds both halves of silu(gate) * up;
//   RESID  : fp32 residual stream += tile;  F32: logits = logit_scale * tile;  STORE.
//
// Kernels:
//   gemm_skinny_bf16 (M <= 64): weight streaming.  Each wave owns 32 weight rows and
//     loads them straight from HBM into MFMA operand registers (16-byte loads, two
//     register sets so the next 128-wide K stage is in flight during the current one);
//     the activation slice is staged once per workgroup in LDS and shared by 4 waves.
//     Split-K over gridDim.y fills the chip; partial tiles go to a workspace and the
//     last workgroup of a tile (device-scope arrival counter) sums them in split order
//     and runs the epilogue: deterministic, no float atomics.
//   gemm_tiled_bf16 (M > 64): 128x128 output tiles, 64-wide K stages double-buffered in
//     LDS with register prefetch, 4 waves each computing 64x64 with 32x32x16 MFMAs; the
//     same split-K machinery for shapes with too few tiles.
//   gemm_f32: SIMT fp32 kernel for fp32 models (32x128 tiles).
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

__device__ __forceinline__ int acc_row(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

// Epilogue over an fp32 tile in LDS: tile[r * ldt + c] is output row m0 + r and virtual
// column vc0 + c (c < 128).
template <typename T, int EPI>
__device__ void epilogue(const float* tile, int ldt, int rows, int m0, int vc0, int M, int Nv,
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
        Elt<T>::store(dst, (int64_t)j * e.Sp + pos, x1);
        Elt<T>::store(dst, (int64_t)(j + half) * e.Sp + pos, x2);
      }
    }
  }
}

// Sum split-K partials [splits][M][Nv] of one tile in split order into the LDS tile.
__device__ __forceinline__ void gather_partials(float* tile, int ldt, int rows, int m0, int vc0,
                                                int M, int Nv, int splits, const float* part) {
  for (int i = threadIdx.x; i < rows * 128; i += blockDim.x) {
    int r = i >> 7, c = i & 127;
    int m = m0 + r, vc = vc0 + c;
    float s = 0.f;
    if (m < M && vc < Nv)
      for (int sp = 0; sp < splits; ++sp) s += part[((int64_t)sp * M + m) * Nv + vc];
    tile[r * ldt + c] = s;
  }
}

// ============================================================================
// skinny bf16 GEMM
// ============================================================================
constexpr int SK_KS = 128;          // K per stage
constexpr int SK_LDX = SK_KS + 8;   // LDS row stride of the activation stage (elements)
constexpr int TL = 132;             // LDS row stride of the fp32 epilogue tile

template <int EPI, int MT>
__global__ __launch_bounds__(256, 2) void gemm_skinny_bf16(
    const uint16_t* __restrict__ X, int ldx, const uint16_t* __restrict__ W, int M, int Nv,
    int K, int kchunk, int splits, float* part, int* counters, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][MT * 32 * SK_LDX];
  __shared__ float tile[MT * 32 * TL];
  __shared__ int flag;
  const int tn = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lr = l & 31, g = l >> 5;
  const int vc = tn * 128 + w * 32 + lr;
  const bool wv = vc < Nv;
  const int wrow = wv ? wrow_of<EPI>(vc, e.F) : 0;
  const int kb = split * kchunk;
  const int ke = min(K, kb + kchunk);
  const int nst = (ke - kb) / SK_KS;
  const uint16_t* wp = W + (int64_t)wrow * K + kb + 8 * g;
  const uint16_t* xp = X + kb;

  constexpr int XV = MT * 2;  // 16-byte activation vectors per thread per stage
  u32x4 xr[XV];
  u32x4 wa[8], wb[8];
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};

  auto load_x = [&](int st) {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      int ee = tid + 256 * i;
      int r = ee >> 4, c8 = ee & 15;
      xr[i] = (r < M) ? *reinterpret_cast<const u32x4*>(xp + (int64_t)r * ldx + st * SK_KS + 8 * c8)
                      : u32x4{};
    }
  };
  auto store_x = [&](uint16_t* xs) {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      int ee = tid + 256 * i;
      int r = ee >> 4, c8 = ee & 15;
      *reinterpret_cast<u32x4*>(&xs[r * SK_LDX + 8 * c8]) = xr[i];
    }
  };
  auto load_w = [&](u32x4* wr, int st) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      wr[t] = wv ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp + st * SK_KS + 16 * t))
                 : u32x4{};
  };
  auto compute = [&](const u32x4* wr, const uint16_t* xs) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        u32x4 a = *reinterpret_cast<const u32x4*>(&xs[(mt * 32 + lr) * SK_LDX + 16 * t + 8 * g]);
        acc[mt] = mfma32(as_bf16x8(a), as_bf16x8(wr[t]), acc[mt]);
      }
  };

  load_w(wa, 0);
  load_x(0);
  store_x(Xs[0]);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    if (st + 1 < nst) { load_w(wb, st + 1); load_x(st + 1); }
    compute(wa, Xs[0]);
    if (st + 1 < nst) store_x(Xs[1]);
    __syncthreads();
    if (st + 1 >= nst) break;
    if (st + 2 < nst) { load_w(wa, st + 2); load_x(st + 2); }
    compute(wb, Xs[1]);
    if (st + 2 < nst) store_x(Xs[0]);
    __syncthreads();
  }

  if (splits == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) tile[(mt * 32 + acc_row(v, g)) * TL + w * 32 + lr] = acc[mt][v];
    __syncthreads();
    epilogue<uint16_t, EPI>(tile, TL, MT * 32, 0, tn * 128, M, Nv, e);
    return;
  }
  if (wv) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        int m = mt * 32 + acc_row(v, g);
        if (m < M) part[((int64_t)split * M + m) * Nv + vc] = acc[mt][v];
      }
  }
  if (!arrive_last(&counters[tn], splits, &flag)) return;
  gather_partials(tile, TL, MT * 32, 0, tn * 128, M, Nv, splits, part);
  __syncthreads();
  epilogue<uint16_t, EPI>(tile, TL, MT * 32, 0, tn * 128, M, Nv, e);
}

// ============================================================================
// tiled bf16 GEMM
// ============================================================================
constexpr int TB_K = 64;
constexpr int TB_LD = TB_K + 8;
constexpr int TB_AB_BYTES = 2 * 2 * 128 * TB_LD * 2;
constexpr int TB_TILE_BYTES = 128 * TL * 4;
constexpr int TB_SMEM = TB_AB_BYTES > TB_TILE_BYTES ? TB_AB_BYTES : TB_TILE_BYTES;

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_tiled_bf16(
    const uint16_t* __restrict__ X, int ldx, const uint16_t* __restrict__ W, int M, int Nv, int K,
    int kchunk, int splits, float* part, int* counters, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[TB_SMEM];
  __shared__ int flag;
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + 2 * 128 * TB_LD;
  float* tile = reinterpret_cast<float*>(smem);
  const int tn = blockIdx.x, tm = blockIdx.y, split = blockIdx.z;
  const int m0 = tm * 128, vc0 = tn * 128;
  const int tid = threadIdx.x;
  const int w = tid >> 6, wm = w >> 1, wn = w & 1, l = tid & 63, lr = l & 31, g = l >> 5;
  const int kb = split * kchunk;
  const int ke = min(K, kb + kchunk);
  const int nst = (ke - kb) / TB_K;

  // loader: element e = tid + 256 i  ->  row e >> 3, 16-byte column e & 7
  const uint16_t* arow[4];
  const uint16_t* brow[4];
  bool av[4], bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int ee = tid + 256 * i;
    int r = ee >> 3, c8 = ee & 7;
    int m = m0 + r, vc = vc0 + r;
    av[i] = m < M;
    bv[i] = vc < Nv;
    arow[i] = X + (int64_t)(av[i] ? m : 0) * ldx + kb + 8 * c8;
    brow[i] = W + (int64_t)(bv[i] ? wrow_of<EPI>(vc, e.F) : 0) * K + kb + 8 * c8;
  }
  u32x4 ra[4], rb[4];
  auto load = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = av[i] ? *reinterpret_cast<const u32x4*>(arow[i] + st * TB_K) : u32x4{};
      rb[i] = bv[i] ? *reinterpret_cast<const u32x4*>(brow[i] + st * TB_K) : u32x4{};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int ee = tid + 256 * i;
      int r = ee >> 3, c8 = ee & 7;
      *reinterpret_cast<u32x4*>(&As[(buf * 128 + r) * TB_LD + 8 * c8]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[(buf * 128 + r) * TB_LD + 8 * c8]) = rb[i];
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

  load(0);
  store(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) load(st + 1);
    compute(st & 1);
    if (st + 1 < nst) store((st + 1) & 1);
    __syncthreads();
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
  for (int i = tid; i < 128 * 128; i += 256) {
    int r = i >> 7, c = i & 127;
    int m = m0 + r, vc = vc0 + c;
    if (m < M && vc < Nv) part[((int64_t)split * M + m) * Nv + vc] = tile[r * TL + c];
  }
  if (!arrive_last(&counters[tm * gridDim.x + tn], splits, &flag)) return;
  gather_partials(tile, TL, 128, m0, vc0, M, Nv, splits, part);
  __syncthreads();
  epilogue<uint16_t, EPI>(tile, TL, 128, m0, vc0, M, Nv, e);
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
// planning and dispatch
// ============================================================================
GemmPlan gemm_plan(int dtype, int M, int Nv, int K) {
  GemmPlan p;
  p.ntn = (Nv + 127) / 128;
  if (dtype == F32) {
    p.kind = GEMM_F32;
    p.ntm = (M + 31) / 32;
    p.kchunk = K;
    return p;
  }
  int ks;
  if (M <= 64) {
    p.kind = GEMM_SKINNY;
    p.mt = (M <= 32) ? 1 : 2;
    p.ntm = 1;
    ks = SK_KS;
  } else {
    p.kind = GEMM_TILED;
    p.ntm = (M + 127) / 128;
    ks = TB_K;
  }
  const int tiles = p.ntn * p.ntm;
  const int target = 512;
  int splits = 1;
  if (tiles < target) {
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
    p.counters = tiles;
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
    dim3 grid(p.ntn, p.splits);
    if (p.mt == 1)
      gemm_skinny_bf16<EPI, 1><<<grid, 256, 0, st>>>((const uint16_t*)X, ldx, (const uint16_t*)W,
                                                      M, Nv, K, p.kchunk, p.splits, part,
                                                      counters, e);
    else
      gemm_skinny_bf16<EPI, 2><<<grid, 256, 0, st>>>((const uint16_t*)X, ldx, (const uint16_t*)W,
                                                      M, Nv, K, p.kchunk, p.splits, part,
                                                      counters, e);
  } else {
    gemm_tiled_bf16<EPI><<<dim3(p.ntn, p.ntm, p.splits), 256, 0, st>>>(
        (const uint16_t*)X, ldx, (const uint16_t*)W, M, Nv, K, p.kchunk, p.splits, part, counters,
        e);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epi, const GemmPlan& p, const void* X, int ldx,
                       const void* W, int M, int Nv, int K, const EpiArgs& e, float* part,
                       int* counters, hipStream_t st) {
  if (M <= 0 || Nv <= 0) return hipSuccess;
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
