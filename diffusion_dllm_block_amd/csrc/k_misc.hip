// Small kernels: RoPE table, embedding gather + RMSNorm, RMSNorm, fills, and the
// device side of the seeded synthetic-input generator.
#include "common.h"
#include "kernels.h"

namespace dllm {

// ------------------------------------------------------------------ RoPE table
// cos/sin [S][D/2] of pos * theta^(-2j/D), evaluated in double, stored fp32.
__global__ void rope_table_kernel(float* cosb, float* sinb, int S, int D, double theta) {
  int half = D / 2;
  int64_t n = (int64_t)S * half;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    int pos = (int)(i / half), j = (int)(i % half);
    double inv = pow(theta, -2.0 * (double)j / (double)D);
    double a = (double)pos * inv;
    cosb[i] = (float)cos(a);
    sinb[i] = (float)sin(a);
  }
}

hipError_t launch_rope_table(float* cosb, float* sinb, int S, int D, float theta, hipStream_t st) {
  int64_t n = (int64_t)S * (D / 2);
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  rope_table_kernel<<<blocks, 256, 0, st>>>(cosb, sinb, S, D, (double)theta);
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm
// One workgroup per row; sum of squares reduced in a fixed order (per-thread
// sequential, wave butterfly, then the 4 waves in order).
template <typename T>
__device__ __forceinline__ void rms_row(const float* xr, const T* g, float eps, int d, T* hr,
                                        float* red) {
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) ss += xr[i] * xr[i];
  ss = wave_sum(ss);
  int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (l == 0) red[w] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < (int)(blockDim.x / kWave); ++i) tot += red[i];
  float r = 1.0f / sqrtf(tot / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += blockDim.x)
    Elt<T>::store(hr, i, (xr[i] * r) * Elt<T>::load(g, i));
}

template <typename T>
__global__ __launch_bounds__(256) void embed_norm_kernel(const int* tokens, int S, int r0, int R,
                                                         const T* embed, const T* g, float eps,
                                                         int d, int V, float* x, T* h) {
  __shared__ float red[4];
  int j = blockIdx.x;
  int b = j / R, i = j % R;
  int tok = tokens[(int64_t)b * S + r0 + i];
  tok = min(max(tok, 0), V - 1);  // ids outside [0, V) are not valid input; never read out of bounds
  const T* er = embed + (int64_t)tok * d;
  float* xr = x + (int64_t)j * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) xr[c] = Elt<T>::load(er, c);
  __syncthreads();
  rms_row<T>(xr, g, eps, d, h + (int64_t)j * d, red);
}

// Single pass, the row held in registers: 1024 threads, thread t owns the float4 columns
// 4t + 4096j (j < NJ; columns >= d are skipped).  x = x + part[0] + ... + part[splits-1]
// (split order), written back; then h = x / sqrt(mean(x^2) + eps) * g.  The loads of up
// to G splits are all issued before the first add, so a typical fold is one memory
// round trip.  Needs d % 4 == 0 and d <= 4096 * NJ.
constexpr int kFoldThreads = 1024;
template <typename T, int NJ, int G>
__global__ __launch_bounds__(kFoldThreads) void fold_norm_kernel(float* x, int Rin, int Kout,
                                                                const T* g, float eps, int d,
                                                                T* h, PartView pv) {
  __shared__ float red[kFoldThreads / kWave];
  const int j0 = blockIdx.x;
  const int in_row = (j0 / Kout) * Rin + (j0 % Kout);
  float* xr = x + (int64_t)in_row * d;
  const int64_t stride = pv.split_stride();
  const int tid = threadIdx.x;
  float4 v[NJ];
  float gv[NJ][4];  // the gains, read together with x and the partials
  bool ok[NJ];
  int col[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    col[j] = 4 * tid + 4096 * j;
    ok[j] = col[j] < d;
    col[j] = ok[j] ? col[j] : 0;  // clamped, never stored
    v[j] = *reinterpret_cast<const float4*>(xr + col[j]);
#pragma unroll
    for (int u = 0; u < 4; ++u) gv[j][u] = Elt<T>::load(g, col[j] + u);
  }
  for (int s0 = 0; s0 < pv.splits; s0 += G) {
    float4 pvv[G][NJ];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int sp = min(s0 + u, pv.splits - 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        pvv[u][j] = *reinterpret_cast<const float4*>(pv.p + sp * stride + pv.off(in_row, col[j]));
    }
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (s0 + u < pv.splits)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          v[j].x += pvv[u][j].x; v[j].y += pvv[u][j].y; v[j].z += pvv[u][j].z; v[j].w += pvv[u][j].w;
        }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (!ok[j]) continue;
    ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    if (pv.splits > 0) *reinterpret_cast<float4*>(xr + col[j]) = v[j];
  }
  ss = wave_sum(ss);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kFoldThreads / kWave; ++i) tot += red[i];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  T* hr = h + (int64_t)j0 * d;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (!ok[j]) continue;
    const int c = col[j];
    const float o0 = (v[j].x * r) * gv[j][0], o1 = (v[j].y * r) * gv[j][1];
    const float o2 = (v[j].z * r) * gv[j][2], o3 = (v[j].w * r) * gv[j][3];
    if constexpr (sizeof(T) == 2) {  // bf16: one 8-byte store
      *reinterpret_cast<u16x4*>(hr + c) = u16x4{f2bf(o0), f2bf(o1), f2bf(o2), f2bf(o3)};
    } else {
      *reinterpret_cast<float4*>(hr + c) = make_float4(o0, o1, o2, o3);
    }
  }
}

// Embedding gather + RMSNorm in one pass, the row in registers (the layout of
// fold_norm_kernel): x[j] = embed[token] (fp32), h[j] = rmsnorm(x[j]) * g.
template <typename T, int NJ>
__global__ __launch_bounds__(kFoldThreads) void embed_norm_fast(const int* tokens, int S, int r0,
                                                               int R, const T* embed, const T* g,
                                                               float eps, int d, int V, float* x,
                                                               T* h) {
  __shared__ float red[kFoldThreads / kWave];
  const int j0 = blockIdx.x;
  const int b = j0 / R, i = j0 % R;
  int tok = tokens[(int64_t)b * S + r0 + i];
  tok = min(max(tok, 0), V - 1);  // ids outside [0, V) are not valid input; never read out of bounds
  const T* er = embed + (int64_t)tok * d;
  const int tid = threadIdx.x;
  float v[NJ][4], gv[NJ][4];
  bool ok[NJ];
  int col[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    col[jj] = 4 * tid + 4096 * jj;
    ok[jj] = col[jj] < d;
    col[jj] = ok[jj] ? col[jj] : 0;  // clamped, never stored
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[jj][u] = Elt<T>::load(er, col[jj] + u);
      gv[jj][u] = Elt<T>::load(g, col[jj] + u);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
    if (ok[jj]) ss += v[jj][0] * v[jj][0] + v[jj][1] * v[jj][1] + v[jj][2] * v[jj][2] + v[jj][3] * v[jj][3];
  ss = wave_sum(ss);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int k = 0; k < kFoldThreads / kWave; ++k) tot += red[k];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  float* xr = x + (int64_t)j0 * d;
  T* hr = h + (int64_t)j0 * d;
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    if (!ok[jj]) continue;
    const int c = col[jj];
    *reinterpret_cast<float4*>(xr + c) = make_float4(v[jj][0], v[jj][1], v[jj][2], v[jj][3]);
    float o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = (v[jj][u] * r) * gv[jj][u];
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<u16x4*>(hr + c) = u16x4{f2bf(o[0]), f2bf(o[1]), f2bf(o[2]), f2bf(o[3])};
    } else {
      *reinterpret_cast<float4*>(hr + c) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(float* x, int Rin, int Kout, const T* g,
                                                      float eps, int d, T* h, PartView pv) {
  __shared__ float red[4];
  int j = blockIdx.x;
  const int in_row = (j / Kout) * Rin + (j % Kout);
  float* xr = x + (int64_t)in_row * d;
  if (pv.splits > 0) {
    // add the pending split-K partials of the residual GEMM, in split order
    const int64_t stride = pv.split_stride();
    for (int c = threadIdx.x; c < d; c += blockDim.x) {
      float v = xr[c];
      for (int s = 0; s < pv.splits; ++s) v += pv.p[s * stride + pv.off(in_row, c)];
      xr[c] = v;
    }
    __syncthreads();
  }
  rms_row<T>(xr, g, eps, d, h + (int64_t)j * d, red);
}

hipError_t launch_embed_norm(int dtype, const int* tokens, int S, int r0, int R, int B,
                             const void* embed, const void* g, float eps, int d, int V, float* x,
                             void* h, hipStream_t st) {
  dim3 grid(B * R);
  if (d % 4 == 0 && d <= 8192) {
#define DLLM_EMB(TT, NJV)                                                                   \
  embed_norm_fast<TT, NJV><<<grid, kFoldThreads, 0, st>>>(tokens, S, r0, R, (const TT*)embed, \
                                                          (const TT*)g, eps, d, V, x, (TT*)h)
    if (dtype == F32) {
      if (d <= 4096) DLLM_EMB(float, 1); else DLLM_EMB(float, 2);
    } else {
      if (d <= 4096) DLLM_EMB(uint16_t, 1); else DLLM_EMB(uint16_t, 2);
    }
#undef DLLM_EMB
    return hipGetLastError();
  }
  if (dtype == F32)
    embed_norm_kernel<float><<<grid, 256, 0, st>>>(tokens, S, r0, R, (const float*)embed,
                                                   (const float*)g, eps, d, V, x, (float*)h);
  else
    embed_norm_kernel<uint16_t><<<grid, 256, 0, st>>>(tokens, S, r0, R, (const uint16_t*)embed,
                                                      (const uint16_t*)g, eps, d, V, x,
                                                      (uint16_t*)h);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, float* x, int rows, int Rin, int Kout, const void* g,
                          float eps, int d, void* h, const PartView& pv, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (d % 4 == 0 && d <= 8192) {
#define DLLM_FOLD(TT, NJV, GV)                                                    \
  fold_norm_kernel<TT, NJV, GV><<<rows, kFoldThreads, 0, st>>>(x, Rin, Kout, (const TT*)g, eps, \
                                                              d, (TT*)h, pv)
    // the group covers the splits with as few redundant (clamped) loads as possible
    const int sp = pv.splits;
    if (dtype == F32) {
      if (d <= 4096) {
        if (sp <= 2) DLLM_FOLD(float, 1, 2); else if (sp <= 4) DLLM_FOLD(float, 1, 4);
        else if (sp <= 8) DLLM_FOLD(float, 1, 8); else DLLM_FOLD(float, 1, 16);
      } else {
        if (sp <= 2) DLLM_FOLD(float, 2, 2); else if (sp <= 4) DLLM_FOLD(float, 2, 4);
        else DLLM_FOLD(float, 2, 8);
      }
    } else {
      if (d <= 4096) {
        if (sp <= 2) DLLM_FOLD(uint16_t, 1, 2); else if (sp <= 4) DLLM_FOLD(uint16_t, 1, 4);
        else if (sp <= 8) DLLM_FOLD(uint16_t, 1, 8); else DLLM_FOLD(uint16_t, 1, 16);
      } else {
        if (sp <= 2) DLLM_FOLD(uint16_t, 2, 2); else if (sp <= 4) DLLM_FOLD(uint16_t, 2, 4);
        else DLLM_FOLD(uint16_t, 2, 8);
      }
    }
#undef DLLM_FOLD
    return hipGetLastError();
  }
  if (dtype == F32)
    rmsnorm_kernel<float><<<rows, 256, 0, st>>>(x, Rin, Kout, (const float*)g, eps, d, (float*)h, pv);
  else
    rmsnorm_kernel<uint16_t><<<rows, 256, 0, st>>>(x, Rin, Kout, (const uint16_t*)g, eps, d,
                                                   (uint16_t*)h, pv);
  return hipGetLastError();
}

template <typename T, int G>
__global__ __launch_bounds__(kFoldSeg / 4) void fold_scale_kernel(float* x, int Rin, int Kout,
                                                                 const T* g, int d, T* h,
                                                                 float* rss, PartView pv) {
  constexpr int NW = kFoldSeg / 4 / kWave;
  __shared__ float red[NW];
  const int j = blockIdx.y, seg = blockIdx.x;
  const int in_row = (j / Kout) * Rin + (j % Kout);
  const int col = seg * kFoldSeg + 4 * (int)threadIdx.x;
  const bool ok = col < d;
  const int c = ok ? col : 0;  // clamped, never stored
  float* xr = x + (int64_t)in_row * d;
  float4 v = *reinterpret_cast<const float4*>(xr + c);
  float gv[4];
  if constexpr (sizeof(T) == 2) {
    const u16x4 gg = *reinterpret_cast<const u16x4*>(g + c);
#pragma unroll
    for (int u = 0; u < 4; ++u) gv[u] = bf2f(gg[u]);
  } else {
    const float4 gg = *reinterpret_cast<const float4*>(g + c);
    gv[0] = gg.x; gv[1] = gg.y; gv[2] = gg.z; gv[3] = gg.w;
  }
  const int64_t stride = pv.split_stride();
  for (int s0 = 0; s0 < pv.splits; s0 += G) {  // all of a group's loads in flight together
    float4 pp[G];
#pragma unroll
    for (int u = 0; u < G; ++u)
      pp[u] = *reinterpret_cast<const float4*>(pv.p + min(s0 + u, pv.splits - 1) * stride +
                                               pv.off(in_row, c));
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (s0 + u < pv.splits) { v.x += pp[u].x; v.y += pp[u].y; v.z += pp[u].z; v.w += pp[u].w; }
  }
  if (ok) {
    if (pv.splits > 0) *reinterpret_cast<float4*>(xr + c) = v;
    const float o0 = v.x * gv[0], o1 = v.y * gv[1], o2 = v.z * gv[2], o3 = v.w * gv[3];
    T* hr = h + (int64_t)j * d + c;
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<u16x4*>(hr) = u16x4{f2bf(o0), f2bf(o1), f2bf(o2), f2bf(o3)};
    } else {
      *reinterpret_cast<float4*>(hr) = make_float4(o0, o1, o2, o3);
    }
  }
  float q = ok ? v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w : 0.f;
  q = wave_sum_dpp(q);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = q;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) t += red[i];
    rss[(int64_t)j * gridDim.x + seg] = t;
  }
}

hipError_t launch_fold_scale(int dtype, float* x, int rows, int Rin, int Kout, const void* g,
                             int d, void* h, float* rss, const PartView& pv, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (d % 4) return hipErrorInvalidValue;
  const dim3 grid((d + kFoldSeg - 1) / kFoldSeg, rows);
#define DLLM_FS(TT, GV)                                                                   \
  fold_scale_kernel<TT, GV><<<grid, kFoldSeg / 4, 0, st>>>(x, Rin, Kout, (const TT*)g, d, \
                                                          (TT*)h, rss, pv)
  // a fixed group of 8: sizing it to the split count (2 for the 8B output projection)
  // measured slower here, unlike in fold_norm_kernel
  if (dtype == F32) DLLM_FS(float, 8);
  else DLLM_FS(uint16_t, 8);
#undef DLLM_FS
  return hipGetLastError();
}

__global__ void fold_partials_kernel(float* y, PartView pv) {
  const int64_t n = (int64_t)pv.M * pv.N;
  const int64_t stride = pv.split_stride();
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / pv.N), c = (int)(i % pv.N);
    float v = y[i];
    for (int s = 0; s < pv.splits; ++s) v += pv.p[s * stride + pv.off(m, c)];
    y[i] = v;
  }
}

hipError_t launch_fold_partials(float* y, const PartView& pv, hipStream_t st) {
  const int64_t n = (int64_t)pv.M * pv.N;
  if (n <= 0 || pv.splits <= 0) return hipSuccess;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  fold_partials_kernel<<<blocks, 256, 0, st>>>(y, pv);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fills
__global__ void fill_i32_kernel(int* p, int64_t n, int v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_i32(int* p, int64_t n, int v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 2048) blocks = 2048;
  fill_i32_kernel<<<blocks, 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

// ------------------------------------------------------------------ synthetic inputs
// SplitMix64 (Steele, Lea and Flood 2014): output i of a stream with state x0 is
// mix(x0 + (i+1) * GAMMA).  Normal deviates by Irwin-Hall over the four 16-bit fields.
__device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <typename T>
__global__ void synth_fill_kernel(T* dst, int64_t n, uint64_t x0, double stdv, int mode) {
#pragma clang fp contract(off)
  const double c = 0x1.bb67ae8584caap+0 / 65536.0;  // sqrt(3) / 2^16
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    double v;
    if (mode == 2) {
      v = stdv;
    } else {
      uint64_t r = sm64_mix(x0 + ((uint64_t)i + 1ull) * 0x9E3779B97F4A7C15ull);
      int64_t s = (int64_t)(r & 0xFFFF) + (int64_t)((r >> 16) & 0xFFFF) +
                  (int64_t)((r >> 32) & 0xFFFF) + (int64_t)(r >> 48) - 131070;
      double z = __dmul_rn((double)s, c);
      v = __dmul_rn(z, stdv);
      if (mode == 1) v = __dadd_rn(1.0, v);
    }
    Elt<T>::store(dst, i, __double2float_rn(v));
  }
}

hipError_t launch_synth_fill(void* dst, int64_t n, int dtype, uint64_t seed, uint32_t tid,
                             double stdv, int mode, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  uint64_t s = seed ^ ((uint64_t)tid << 32);
  // first output of a SplitMix64 stream seeded with s (computed on the host)
  uint64_t z = s + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  uint64_t x0 = z ^ (z >> 31);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (dtype == F32)
    synth_fill_kernel<float><<<(int)blocks, 256, 0, st>>>((float*)dst, n, x0, stdv, mode);
  else
    synth_fill_kernel<uint16_t><<<(int)blocks, 256, 0, st>>>((uint16_t*)dst, n, x0, stdv, mode);
  return hipGetLastError();
}

// ------------------------------------------------------------------ cache staleness
// How far the block-wise approximate cache is from the exact K/V of the current tokens:
// the pages report that the K/V activations of adjacent denoising steps have a cosine
// similarity close to 1, which is what makes reusing them safe (ccyt168.com Fast-dLLM
// article, section 1.1, the similarity check; techwalker.com explainer, "Core
// innovation").  Pass 1, grid (B*Hkv, 2, L): one (sequence, KV head) of one layer's K
// (y = 0) or V (y = 1); wave w takes positions w, w + 4, ... outside [x0, x1), the
// cosine similarity of the cached and fresh D-vectors in fp32 (both zero: 1, one zero:
// 0), summed in double and minimised per wave, then over the 4 waves in order.
template <typename T>
__global__ __launch_bounds__(256) void staleness_partials_kernel(
    const T* __restrict__ cached, const T* __restrict__ fresh, int B, int Hkv, int S, int Sp,
    int D, int x0, int x1, double* part) {
  __shared__ double rsum[4], rcnt[4];
  __shared__ float rmin[4];
  const int bh = blockIdx.x, kv = blockIdx.y, l = blockIdx.z;
  const int64_t per = (int64_t)B * Hkv * Sp * D;  // elements of K (= of Vt) per layer
  const int64_t base = (int64_t)l * 2 * per + kv * per + (int64_t)bh * Sp * D;
  const T* a = cached + base;
  const T* f = fresh + base;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double sum = 0.0, cnt = 0.0;
  float mn = INFINITY;
  for (int p = w; p < S; p += 4) {
    if (p >= x0 && p < x1) continue;  // uniform over the wave
    float dot = 0.f, na = 0.f, nb = 0.f;
    for (int d = lane; d < D; d += kWave) {
      const int64_t o = kv == 0 ? (int64_t)p * D + d : vt_off(d, p, D);
      const float u = Elt<T>::load(a, o), v = Elt<T>::load(f, o);
      dot += u * v;
      na += u * u;
      nb += v * v;
    }
    dot = wave_sum_dpp(dot);
    na = wave_sum_dpp(na);
    nb = wave_sum_dpp(nb);
    const float c = (na == 0.f && nb == 0.f) ? 1.f
                    : (na == 0.f || nb == 0.f) ? 0.f
                    : dot / sqrtf(na * nb);
    sum += c;
    cnt += 1.0;
    mn = fminf(mn, c);
  }
  if (lane == 0) { rsum[w] = sum; rcnt[w] = cnt; rmin[w] = mn; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0, n = 0.0;
    float m = INFINITY;
    for (int i = 0; i < 4; ++i) { s += rsum[i]; n += rcnt[i]; m = fminf(m, rmin[i]); }
    double* o = part + ((int64_t)(l * 2 + kv) * gridDim.x + bh) * 3;
    o[0] = s;
    o[1] = n;
    o[2] = (double)m;
  }
}

// Pass 2, one thread per (layer, K or V): the (sequence, head) partials in order; out
// [L][2][2] = mean, min (1, 1 when no position is compared).
__global__ void staleness_final_kernel(const double* part, int nbh, int n, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double* p = part + (int64_t)i * nbh * 3;
  double s = 0.0, c = 0.0, m = INFINITY;
  for (int j = 0; j < nbh; ++j) {
    s += p[3 * j];
    c += p[3 * j + 1];
    m = fmin(m, p[3 * j + 2]);
  }
  out[2 * i] = c > 0.0 ? (float)(s / c) : 1.f;
  out[2 * i + 1] = c > 0.0 ? (float)m : 1.f;
}

hipError_t launch_staleness(int dtype, const void* cached, const void* fresh, int L, int B,
                            int Hkv, int S, int Sp, int D, int x0, int x1, double* part,
                            float* out, hipStream_t st) {
  if (L <= 0 || B <= 0 || Hkv <= 0) return hipSuccess;
  const dim3 grid(B * Hkv, 2, L);
  if (dtype == F32)
    staleness_partials_kernel<float><<<grid, 256, 0, st>>>((const float*)cached, (const float*)fresh,
                                                           B, Hkv, S, Sp, D, x0, x1, part);
  else
    staleness_partials_kernel<uint16_t><<<grid, 256, 0, st>>>(
        (const uint16_t*)cached, (const uint16_t*)fresh, B, Hkv, S, Sp, D, x0, x1, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n = L * 2;
  staleness_final_kernel<<<(n + 63) / 64, 64, 0, st>>>(part, B * Hkv, n, out);
  return hipGetLastError();
}

}  // namespace dllm
