// Non-causal attention of query rows against the per-layer KV cache.
//
// A masked-diffusion LLM attends bidirectionally: every query sees every position,
// so there is no causal mask (ccyt168.com Fast-dLLM article, section 1.1 "Block-Wise
// KV Cache"; techwalker.com explainer, "Core innovation: a KV cache suited to diffusion
// models").  During a cached step the block's queries read the cached K/V of all S
// positions (their own rows freshly written); during a refresh every row is a query.
//
// Cache layout: K [B][Hkv][Sp][D] and V transposed, Vt [B][Hkv][D][Sp].  With both
// products written transposed,
//     S^T = K . Q^T     (A = K rows, B = Q rows: 16-byte row loads for both)
//     O^T = Vt . P^T    (A = Vt rows, B = P taken straight from the S^T accumulator)
// each lane of a 32x32 MFMA tile owns one query column in both products, so the
// online-softmax statistics of a query live in one lane pair (l, l^32) and P never
// needs a shuffle or an LDS round trip.
//
// bf16 MFMA layout used (v_mfma_f32_32x32x16_bf16, wave64): lane l, half g = l/32:
//   A: row l%32, k = 8g..8g+7;  B: column l%32, k = 8g..8g+7;
//   C: column l%32, rows 8*(v/4) + 4g + (v%4) for accumulator element v = 0..15.
// Any consistent k permutation is valid for A and B; the P^T operand uses the
// accumulator's own row order, and the Vt operand reads the same keys.
#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int HD = 128;  // head dim of the bf16 MFMA kernels

// key offset (within a 32-key tile) held by accumulator element v of half g
__device__ __forceinline__ int acc_row(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

// Pack accumulator elements 8u..8u+7 (as bf16) into an MFMA operand.
__device__ __forceinline__ bf16x8 pack_p(const float* p, int u) {
  u16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = f2bf(p[8 * u + e]);
  return __builtin_bit_cast(bf16x8, r);
}

// Vt operand for keys {16u + 4g + 0..3, 16u + 8 + 4g + 0..3} of a 32-key tile at key0,
// row d; keys >= S read as zero.
__device__ __forceinline__ bf16x8 load_vt(const uint16_t* vrow, int key0, int u, int g, int S) {
  int ka = key0 + 16 * u + 4 * g;
  int kb = ka + 8;
  u32x2 a = u32x2{}, b = u32x2{};
  if (ka < S) a = *reinterpret_cast<const u32x2*>(vrow + ka);
  if (kb < S) b = *reinterpret_cast<const u32x2*>(vrow + kb);
  if (ka + 4 > S) {  // partial run at the end of the sequence
    uint16_t* pa = reinterpret_cast<uint16_t*>(&a);
    for (int e = 0; e < 4; ++e) if (ka + e >= S) pa[e] = 0;
  }
  if (kb + 4 > S) {
    uint16_t* pb = reinterpret_cast<uint16_t*>(&b);
    for (int e = 0; e < 4; ++e) if (kb + e >= S) pb[e] = 0;
  }
  u32x4 r = u32x4{a.x, a.y, b.x, b.y};
  return as_bf16x8(r);
}

// ============================================================================
// Split-KV attention for a few query rows (a block step): grid (nchunk, Hq*nqt, B),
// 4 waves; wave w covers keys chunk*128 + w*32 .. +32 for a tile of 32 query rows.
// ============================================================================
__global__ __launch_bounds__(256, 2) void attn_splitkv_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, uint16_t* __restrict__ o, int Hq, int Hkv, int R, int S,
    int Sp, int nqt, int nchunk, float scale_log2, float* part_o, float* part_ml,
    int* counters) {
  __shared__ float red_m[4][32], red_l[4][32];
  __shared__ float osum[HD][33];
  __shared__ int flag;
  const int chunk = blockIdx.x;
  const int hq = blockIdx.y / nqt, qt = blockIdx.y % nqt, b = blockIdx.z;
  const int hkv = hq / (Hq / Hkv);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, lr = l & 31, g = l >> 5;
  const int key0 = chunk * 128 + w * 32;

  // Q^T operand: lane (query lr, half g) holds Q[row][16t + 8g .. +8]
  const int qrow = qt * 32 + lr;
  const uint16_t* qp = q + (((int64_t)b * Hq + hq) * R + qrow) * HD + 8 * g;
  u32x4 qf[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
    qf[t] = (qrow < R) ? *reinterpret_cast<const u32x4*>(qp + 16 * t) : u32x4{};
  // K operand: lane (key lr, half g)
  const int key = key0 + lr;
  const uint16_t* kp = k + (((int64_t)b * Hkv + hkv) * Sp + key) * HD + 8 * g;
  u32x4 kf[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
    kf[t] = (key < S) ? *reinterpret_cast<const u32x4*>(kp + 16 * t) : u32x4{};
  // Vt operands: rows d = 32*dt + lr
  const uint16_t* vbase = vt + ((int64_t)b * Hkv + hkv) * HD * Sp;
  bf16x8 vf[4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      vf[dt][u] = load_vt(vbase + (int64_t)(32 * dt + lr) * Sp, key0, u, g, S);

  f32x16 s = {};
#pragma unroll
  for (int t = 0; t < 8; ++t) s = mfma32(as_bf16x8(kf[t]), as_bf16x8(qf[t]), s);

  float p[16];
  float mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float x = (key0 + acc_row(v, g) < S) ? s[v] * scale_log2 : -INFINITY;
    p[v] = x;
    mx = fmaxf(mx, x);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  const float ms = (mx == -INFINITY) ? 0.f : mx;
  float ls = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    p[v] = __builtin_amdgcn_exp2f(p[v] - ms);
    ls += p[v];
  }
  ls += __shfl_xor(ls, 32, kWave);

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    oacc[dt] = f32x16{};
#pragma unroll
    for (int u = 0; u < 2; ++u) oacc[dt] = mfma32(vf[dt][u], pack_p(p, u), oacc[dt]);
  }

  // ---- merge the 4 waves (fixed order)
  if (g == 0) { red_m[w][lr] = mx; red_l[w][lr] = ls; }
  __syncthreads();
  float M = red_m[0][lr];
  for (int i = 1; i < 4; ++i) M = fmaxf(M, red_m[i][lr]);
  float L = 0.f;
  for (int i = 0; i < 4; ++i)
    L += (red_m[i][lr] == -INFINITY) ? 0.f : red_l[i][lr] * __builtin_amdgcn_exp2f(red_m[i][lr] - M);
  const float f = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mx - M);
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int d = 32 * dt + acc_row(v, g);
          float val = oacc[dt][v] * f;
          osum[d][lr] = (ww == 0) ? val : osum[d][lr] + val;
        }
    }
    __syncthreads();
  }

  const int64_t grp = ((int64_t)b * Hq + hq) * nqt + qt;
  if (nchunk == 1) {
    // L per query lives in lanes; publish it through LDS (all reads of red_l are done)
    if (w == 0 && g == 0) red_l[0][lr] = L;
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * HD; e += blockDim.x) {
      int qi = e / HD, d = e % HD;
      int row = qt * 32 + qi;
      if (row < R)
        o[((int64_t)b * R + row) * (Hq * HD) + hq * HD + d] = f2bf(osum[d][qi] / red_l[0][qi]);
    }
    return;
  }

  // ---- publish this chunk's partial (m, l, O) and let the last chunk combine
  float* po = part_o + (grp * nchunk + chunk) * (32 * HD);
  for (int e = threadIdx.x; e < 32 * HD; e += blockDim.x) {
    int qi = e / HD, d = e % HD;
    po[e] = osum[d][qi];
  }
  if (w == 0 && g == 0) {
    float* pml = part_ml + (grp * nchunk + chunk) * 64;
    pml[lr] = M;
    pml[32 + lr] = L;
  }
  if (!arrive_last(&counters[grp], nchunk, &flag)) return;

  // combine chunks in order; thread handles query qi = e / HD for its elements
  for (int e = threadIdx.x; e < 32 * HD; e += blockDim.x) {
    int qi = e / HD, d = e % HD;
    int row = qt * 32 + qi;
    if (row >= R) continue;
    const float* pml = part_ml + grp * nchunk * 64;
    float Mx = -INFINITY;
    for (int c = 0; c < nchunk; ++c) Mx = fmaxf(Mx, pml[c * 64 + qi]);
    float Ls = 0.f, acc = 0.f;
    for (int c = 0; c < nchunk; ++c) {
      float fc = __builtin_amdgcn_exp2f(pml[c * 64 + qi] - Mx);
      Ls += pml[c * 64 + 32 + qi] * fc;
      acc += part_o[(grp * nchunk + c) * (32 * HD) + e] * fc;
    }
    o[((int64_t)b * R + row) * (Hq * HD) + hq * HD + d] = f2bf(acc / Ls);
  }
}

// ============================================================================
// Flash attention over all rows (refresh, or prefix-mode steps with many rows):
// grid (ceil(R/128), Hq, B); wave w owns query rows qt*128 + w*32 .. +32; key tiles of
// 64 staged in LDS and shared by the 4 waves; online softmax per query lane.
// ============================================================================
constexpr int FK = 64;            // keys per LDS tile
constexpr int KS_LD = HD + 8;     // K tile row stride (elements)
constexpr int VS_LD = FK + 8;     // Vt tile row stride (elements)

__global__ __launch_bounds__(256, 2) void attn_flash_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, uint16_t* __restrict__ o, int Hq, int Hkv, int R, int S,
    int Sp, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[FK * KS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[HD * VS_LD];
  const int qt = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int hkv = hq / (Hq / Hkv);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, lr = l & 31, g = l >> 5;
  const int qrow = qt * 128 + w * 32 + lr;

  const uint16_t* qp = q + (((int64_t)b * Hq + hq) * R + qrow) * HD + 8 * g;
  u32x4 qf[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
    qf[t] = (qrow < R) ? *reinterpret_cast<const u32x4*>(qp + 16 * t) : u32x4{};

  const uint16_t* kb = k + ((int64_t)b * Hkv + hkv) * Sp * HD;
  const uint16_t* vb = vt + ((int64_t)b * Hkv + hkv) * HD * Sp;

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int ntile = (S + FK - 1) / FK;
  for (int kt = 0; kt < ntile; ++kt) {
    const int kbase = kt * FK;
    __syncthreads();
    // stage K tile: 64 rows x 128 -> 1024 x 16B, 4 per thread
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = threadIdx.x + 256 * i;
      int r = e >> 4, c8 = e & 15;
      u32x4 val = u32x4{};
      if (kbase + r < S) val = *reinterpret_cast<const u32x4*>(kb + (int64_t)(kbase + r) * HD + 8 * c8);
      *reinterpret_cast<u32x4*>(&Ks[r * KS_LD + 8 * c8]) = val;
    }
    // stage Vt tile: 128 rows x 64 keys -> 1024 x 16B, 4 per thread
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = threadIdx.x + 256 * i;
      int r = e >> 3, c8 = e & 7;
      int kk = kbase + 8 * c8;
      u32x4 val = u32x4{};
      if (kk + 8 <= S) {
        val = *reinterpret_cast<const u32x4*>(vb + (int64_t)r * Sp + kk);
      } else if (kk < S) {
        uint16_t tmp[8];
        for (int e2 = 0; e2 < 8; ++e2) tmp[e2] = (kk + e2 < S) ? vb[(int64_t)r * Sp + kk + e2] : 0;
        val = *reinterpret_cast<u32x4*>(tmp);
      }
      *reinterpret_cast<u32x4*>(&Vs[r * VS_LD + 8 * c8]) = val;
    }
    __syncthreads();

    float p[2][16];
    float tmax = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 s = {};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        u32x4 kv = *reinterpret_cast<const u32x4*>(&Ks[(st * 32 + lr) * KS_LD + 16 * t + 8 * g]);
        s = mfma32(as_bf16x8(kv), as_bf16x8(qf[t]), s);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = (kbase + st * 32 + acc_row(v, g) < S) ? s[v] * scale_log2 : -INFINITY;
        p[st][v] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);   // finite: every tile has a valid key
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float ls = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[st][v] = __builtin_amdgcn_exp2f(p[st][v] - m_new);
        ls += p[st][v];
      }
    ls += __shfl_xor(ls, 32, kWave);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 pb = pack_p(p[st], u);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const uint16_t* vr = &Vs[(32 * dt + lr) * VS_LD + st * 32 + 16 * u + 4 * g];
          u32x2 a = *reinterpret_cast<const u32x2*>(vr);
          u32x2 c = *reinterpret_cast<const u32x2*>(vr + 8);
          bf16x8 va = as_bf16x8(u32x4{a.x, a.y, c.x, c.y});
          oacc[dt] = mfma32(va, pb, oacc[dt]);
        }
      }
  }

  if (qrow < R) {
    const float inv = 1.0f / l_run;
    uint16_t* orow = o + ((int64_t)b * R + qrow) * (Hq * HD) + hq * HD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        // accumulator elements 4*v4 .. 4*v4+3 are d = 32dt + 8*v4 + 4g + 0..3
        u16x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = f2bf(oacc[dt][4 * v4 + e] * inv);
        *reinterpret_cast<u16x4*>(orow + 32 * dt + 8 * v4 + 4 * g) = r;
      }
  }
}

// ============================================================================
// fp32 attention (any D <= 128, modest S): one workgroup per (query row, head, batch).
// ============================================================================
__global__ __launch_bounds__(128) void attn_f32(const float* __restrict__ q,
                                                const float* __restrict__ k,
                                                const float* __restrict__ vt,
                                                float* __restrict__ o, int Hq, int Hkv, int R,
                                                int S, int Sp, int D, float scale) {
  extern __shared__ float sh[];
  float* sc = sh;          // [S]
  float* qs = sh + S;      // [D]
  __shared__ float red[2];
  const int row = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int hkv = hq / (Hq / Hkv);
  const float* qr = q + (((int64_t)b * Hq + hq) * R + row) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) qs[d] = qr[d];
  __syncthreads();
  const float* kb = k + ((int64_t)b * Hkv + hkv) * Sp * D;
  for (int j = threadIdx.x; j < S; j += blockDim.x) {
    float a = 0.f;
    for (int d = 0; d < D; ++d) a += qs[d] * kb[(int64_t)j * D + d];
    sc[j] = a * scale;
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < S; j += blockDim.x) mx = fmaxf(mx, sc[j]);
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  __syncthreads();
  float sum = 0.f;
  for (int j = threadIdx.x; j < S; j += blockDim.x) {
    float e = expf(sc[j] - mx);
    sc[j] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
  __syncthreads();
  sum = red[0] + red[1];
  const float* vb = vt + ((int64_t)b * Hkv + hkv) * D * Sp;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float a = 0.f;
    for (int j = 0; j < S; ++j) a += sc[j] * vb[(int64_t)d * Sp + j];
    o[((int64_t)b * R + row) * (Hq * D) + hq * D + d] = a / sum;
  }
}

AttnPlan attn_plan(int dtype, int B, int Hq, int R, int S, int D) {
  AttnPlan p;
  if (dtype == F32) { p.kind = 0; return p; }
  if (R <= 64) {
    p.kind = 1;
    p.nqt = (R + 31) / 32;
    p.nchunk = (S + 127) / 128;
    if (p.nchunk > 1) {
      p.part_floats = (size_t)B * Hq * p.nqt * p.nchunk * (32 * HD + 64);
      p.counters = B * Hq * p.nqt;
    }
  } else {
    p.kind = 2;
    p.nqt = (R + 127) / 128;
  }
  return p;
}

hipError_t launch_attention(int dtype, const AttnPlan& p, const void* q, const void* k,
                            const void* vt, void* o, int B, int Hq, int Hkv, int R, int S, int Sp,
                            int D, float* part, int* counters, hipStream_t st) {
  if (B <= 0 || R <= 0) return hipSuccess;
  if (p.kind == 0) {
    size_t sh = (size_t)(S + D) * sizeof(float);
    attn_f32<<<dim3(R, Hq, B), 128, sh, st>>>((const float*)q, (const float*)k,
                                                (const float*)vt, (float*)o, Hq, Hkv, R, S, Sp,
                                                D, 1.0f / sqrtf((float)D));
    return hipGetLastError();
  }
  const float scale_log2 = kLog2e / sqrtf((float)D);
  if (p.kind == 1) {
    float* part_o = part;
    float* part_ml = part + (size_t)B * Hq * p.nqt * p.nchunk * (32 * HD);
    attn_splitkv_bf16<<<dim3(p.nchunk, Hq * p.nqt, B), 256, 0, st>>>(
        (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)vt, (uint16_t*)o, Hq, Hkv, R,
        S, Sp, p.nqt, p.nchunk, scale_log2, part_o, part_ml, counters);
  } else {
    attn_flash_bf16<<<dim3(p.nqt, Hq, B), 256, 0, st>>>(
        (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)vt, (uint16_t*)o, Hq, Hkv, R,
        S, Sp, scale_log2);
  }
  return hipGetLastError();
}

}  // namespace dllm
