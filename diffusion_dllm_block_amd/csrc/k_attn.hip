// Non-causal attention of query rows against the per-layer KV cache.
//
// A masked-diffusion LLM attends bidirectionally: every query sees every position,
// so there is no causal mask (ccyt168.com Fast-dLLM article, section 1.1 "Block-Wise
// KV Cache"; techwalker.com explainer, "Core innovation: a KV cache suited to diffusion
// models").  During a cached step the block's queries read the cached K/V of all S
// positions (their own rows freshly written); during a refresh every row is a query.
//
// Cache layout: K [B][Hkv][Sp][D] and V transposed in blocks of 32 keys, Vt
// [B][Hkv][Sp/32][D][32] (vt_off): the 32 keys of a sub-tile are one contiguous 8 KB
// block for D = 128, where a plain [D][Sp] layout spreads them over D rows Sp apart.
// With both products written transposed,
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
#include <algorithm>

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

// 8 bf16 of dim d at keys k..k+7 (k % 8 == 0) of one (sequence, KV head)'s Vt: one
// 16-byte load from a clamped key (Sp % 32 == 0, so every key below S is read from its
// own place and the 8 keys never straddle a 32-key block) ...
__device__ __forceinline__ u32x4 load8_raw(const uint16_t* vb, int d, int k, int Sp) {
  return *reinterpret_cast<const u32x4*>(vb + vt_off(d, min(k, Sp - 8), HD));
}
// ... and, where the 8 keys may reach S, the keys >= S zeroed (n = S - k).  The mask is
// applied where the value is used, not right after the load: masking at the load would
// make the wave wait for a prefetch it does not need yet.
__device__ __forceinline__ u32x4 mask8(const u32x4& v, int n) {
  auto keep = [](int c) {  // c elements of 4 kept
    return c >= 4 ? ~0ull : (c <= 0 ? 0ull : (1ull << (16 * c)) - 1ull);
  };
  const uint64_t lo = (((uint64_t)v[1] << 32) | v[0]) & keep(n);
  const uint64_t hi = (((uint64_t)v[3] << 32) | v[2]) & keep(n - 4);
  return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}

// ============================================================================
// Split-KV attention for a few query rows (a block step): grid (nchunk, Hq*nqt, B),
// NW waves (4 or 8), 32 query rows per workgroup.  Chunk c covers keys
// [c*NW*kpw, (c+1)*NW*kpw); wave w walks its kpw keys in 32-key sub-tiles with an online
// softmax, loading the next sub-tile while the current one is in the MFMAs.
//
// Products use v_mfma_f32_16x16x32_bf16 (lane l: A row l%16, k 8(l/16)..+7; B column
// l%16, same k; C column l%16, rows 4(l/16)+r), so every operand load is 4 lanes x 16
// bytes = 64 contiguous bytes of one K row or one Vt row:
//   S^T tile tau (16 keys x 16 queries) = K . Q^T over 4 k-steps of 32 dims; A row i of
//       tile tau is key 8(i/4) + 4 tau + i%4 of the sub-tile, so lane group j = l/16
//       ends up holding scores of keys 8j .. 8j+7 (tau 0: +0..3, tau 1: +4..7);
//   O^T (16 dims x 16 queries) += Vt . P^T with k = the 32 keys in natural order: the
//       lane's 8 scores are exactly its B operand, and the Vt operand of lane (d, j) is
//       keys 8j .. 8j+7 of row d.
// A query's 32 keys live in the 4 lanes l%16 + 16j, so its max and sum need two partner
// combines (lane ^ 16, lane ^ 32).  The waves are merged through LDS in a fixed order
// (the upper half of the waves hands its rescaled O to the lower half, which adds it
// and publishes the sums).  With several chunks the workgroup writes its unnormalised
// chunk result (O, m, l) and attn_combine merges the chunks in chunk order.
// ============================================================================
constexpr int SK_OLD = HD + 4;  // LDS row stride (floats) of the per-wave O tiles
constexpr int QS_LD = HD + 8;   // LDS row stride (elements) of the staged Q tile

struct KVTile16 {
  u32x4 k[2][4];  // [tau][k-step]: K row of key 8(i/4) + 4 tau + i%4, dims 32 s + 8j
  u32x4 v[8];     // [d-tile]: Vt row 16 dt + l%16, keys 8j .. 8j+7 (unmasked)
};

__device__ __forceinline__ void load_kv16(KVTile16& t, const uint16_t* kbase,
                                          const uint16_t* vbase, int key0, int li, int j, int S,
                                          int Sp) {
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    // keys >= S: any valid K row will do (their scores are masked to -inf)
    const int key = min(key0 + 8 * (li >> 2) + 4 * tau + (li & 3), S - 1);
    const uint16_t* kp = kbase + (int64_t)key * HD + 8 * j;
#pragma unroll
    for (int st = 0; st < 4; ++st) t.k[tau][st] = *reinterpret_cast<const u32x4*>(kp + 32 * st);
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) t.v[dt] = load8_raw(vbase, 16 * dt + li, key0 + 8 * j, Sp);
}

// Chunk partial of one group: O [32][HD] unnormalised (scaled to the chunk maximum m) in
// bf16, then m [32] and l [32] in fp32: kPartStride floats per (group, chunk), m at float
// kPartML.  The bf16 O halves the bytes the chunk kernels write and attn_combine reads
// back (relative rounding 2^-9 per partial, as for the bf16 output itself).
constexpr int kPartML = 32 * HD / 2;
constexpr int kPartStride = kPartML + 64;

__device__ __forceinline__ void part_store_o(float* pc, int qi, int d, float a0, float a1,
                                             float a2, float a3) {
  *reinterpret_cast<u16x4*>(reinterpret_cast<uint16_t*>(pc) + qi * HD + d) =
      u16x4{f2bf(a0), f2bf(a1), f2bf(a2), f2bf(a3)};
}

// The products of one 32-key sub-tile (keys key0 ..) for 32 query rows (two 16-row tiles;
// lane (l%16, j = l/16)), folded into the rows' online-softmax state (O^T unnormalised,
// running maximum m and sum l, in the base-2 exponent domain of scale_log2).
__device__ __forceinline__ void consume_subtile(const KVTile16& t, int key0,
                                                const u32x4 (&qf)[2][4], f32x4 (&oacc)[2][8],
                                                float (&m_run)[2], float (&l_run)[2], int S,
                                                float scale_log2, int j) {
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    f32x4 sc[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      sc[tau] = f32x4{};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        sc[tau] = mfma16(as_bf16x8(t.k[tau][st]), as_bf16x8(qf[qq][st]), sc[tau]);
    }
    // lane's 8 scores: keys key0 + 8j + e, e = 4 tau + r
    float p[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (key0 + 8 * j + e < S) ? sc[e >> 2][e & 3] * scale_log2 : -INFINITY;
      p[e] = x;
      mx = fmaxf(mx, x);
    }
    mx = xor32_combine(xor16_combine(mx, fmax_op), fmax_op);
    const float m_new = fmaxf(m_run[qq], mx);
    // a sub-tile with no valid key at all leaves the state unchanged
    const float alpha = (m_new == -INFINITY || m_run[qq] == -INFINITY)
                            ? ((m_new == -INFINITY) ? 1.f : 0.f)
                            : __builtin_amdgcn_exp2f(m_run[qq] - m_new);
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = (m_new == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(p[e] - m_new);
      ls += p[e];
    }
    ls = xor32_combine(xor16_combine(ls, add_op), add_op);
    l_run[qq] = l_run[qq] * alpha + ls;
    m_run[qq] = m_new;
    u16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = f2bf(p[e]);
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pb);
    // keys >= S: their P is 0, and their Vt values (read from clamped or padding
    // positions) are zeroed so that no stale NaN/Inf reaches the product
    const bool tail = key0 + 32 > S;  // uniform over the wave
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      oacc[qq][dt] *= alpha;
      const u32x4 vv = tail ? mask8(t.v[dt], S - (key0 + 8 * j)) : t.v[dt];
      oacc[qq][dt] = mfma16(as_bf16x8(vv), pop, oacc[qq][dt]);
    }
  }
}

// Plans with a single sub-tile per wave run attn_splitkv_ds_bf16 below instead.
template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_splitkv_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, uint16_t* __restrict__ o, int Hq, int Hkv, int R, int S,
    int Sp, int nqt, int nchunk, int nsub, float scale_log2, float* __restrict__ part) {
  constexpr int NT = NW * 64, NH = 4;  // NH: per-wave O slots in LDS
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  __shared__ float red_m[NW][32], red_l[NW][32];
  __shared__ __attribute__((aligned(16))) float osum[NH][32][SK_OLD];
  const int chunk = blockIdx.x;
  const int hq = blockIdx.y / nqt, qt = blockIdx.y % nqt, b = blockIdx.z;
  const int hkv = hq / (Hq / Hkv);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, li = l & 15, j = l >> 4;
  const int kpw = 32 * nsub;
  const int wkey0 = chunk * NW * kpw + w * kpw;

  // The workgroup's Q tile (32 rows x 128) is read from memory once, 512 16-byte pieces
  // over the workgroup (rows >= R clamped: computed, never stored), issued before the
  // first K/Vt tile so that both are in flight together, then staged in LDS for the
  // waves.  The staging area is the start of osum, which is written only after the
  // products.
  constexpr int QP = 512 / NT;  // Q pieces per thread
  const uint16_t* qh = q + ((int64_t)b * Hq + hq) * R * HD;
  u32x4 qg[QP];
#pragma unroll
  for (int u = 0; u < QP; ++u) {
    const int e = threadIdx.x + NT * u;
    qg[u] = *reinterpret_cast<const u32x4*>(qh + (int64_t)min(qt * 32 + (e >> 4), R - 1) * HD +
                                            8 * (e & 15));
  }
  const uint16_t* kbase = k + ((int64_t)b * Hkv + hkv) * Sp * HD;
  const uint16_t* vbase = vt + ((int64_t)b * Hkv + hkv) * HD * Sp;
  KVTile16 ta;
  load_kv16(ta, kbase, vbase, wkey0, li, j, S, Sp);
  uint16_t* qs = reinterpret_cast<uint16_t*>(&osum[0][0][0]);  // [32][QS_LD]
#pragma unroll
  for (int u = 0; u < QP; ++u) {
    const int e = threadIdx.x + NT * u;
    *reinterpret_cast<u32x4*>(&qs[(e >> 4) * QS_LD + 8 * (e & 15)]) = qg[u];
  }
  __syncthreads();
  // Q^T operands: [query tile qq][k-step]: query 16 qq + li, dims 32 s + 8j .. +8
  u32x4 qf[2][4];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int st = 0; st < 4; ++st)
      qf[qq][st] = *reinterpret_cast<const u32x4*>(&qs[(16 * qq + li) * QS_LD + 8 * j + 32 * st]);

  f32x4 oacc[2][8];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[qq][dt] = f32x4{};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  auto consume = [&](const KVTile16& t, int key0) {
    consume_subtile(t, key0, qf, oacc, m_run, l_run, S, scale_log2, j);
  };

  {
    // The next sub-tile is always requested, past the end too (clamped addresses, never
    // consumed): with no load under a branch, the wait before each consume counts only
    // the sub-tile it needs, and the following one stays in flight.
    // A do-while: a loop that may run zero times lets the compiler sink the first
    // sub-tile's loads (issued above, before the Q tile's LDS store) below the barrier,
    // behind a test on nsub.  The plan gives every wave nsub >= 1; a first sub-tile with
    // no key below S would be all masked and leave the state unchanged.
    KVTile16 tb;
    int n = 0;
    do {
      load_kv16(tb, kbase, vbase, wkey0 + 32 * (n + 1), li, j, S, Sp);
      consume(ta, wkey0 + 32 * n);
      load_kv16(ta, kbase, vbase, wkey0 + 32 * (n + 2), li, j, S, Sp);
      if (n + 1 < nsub) consume(tb, wkey0 + 32 * (n + 1));
      n += 2;
    } while (n < nsub);
  }

  // ---- merge the NW waves (fixed order)
  if (j == 0) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) { red_m[w][16 * qq + li] = m_run[qq]; red_l[w][16 * qq + li] = l_run[qq]; }
  }
  __syncthreads();  // also: every wave is done reading the Q tile staged in osum
  // this wave's O scaled to the workgroup maximum: lane holds query 16 qq + li,
  // dims 16 dt + 4j + r
  float f[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int qi = 16 * qq + li;
    float M = red_m[0][qi];
#pragma unroll
    for (int i = 1; i < NW; ++i) M = fmaxf(M, red_m[i][qi]);
    f[qq] = (m_run[qq] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[qq] - M);
  }
  // eight waves: the upper half hands its O to the lower half (wave w + 4 to wave w),
  // which then publishes the pair's sum; four waves publish their own O directly
  if (w >= NW - NH) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<float4*>(&osum[w - (NW - NH)][16 * qq + li][16 * dt + 4 * j]) =
            make_float4(oacc[qq][dt][0] * f[qq], oacc[qq][dt][1] * f[qq],
                        oacc[qq][dt][2] * f[qq], oacc[qq][dt][3] * f[qq]);
  }
  if constexpr (NW == 8) __syncthreads();
  if (NW == 8 && w < NH) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        float* sp = &osum[w][16 * qq + li][16 * dt + 4 * j];
        const float4 u = *reinterpret_cast<const float4*>(sp);
        *reinterpret_cast<float4*>(sp) =
            make_float4(oacc[qq][dt][0] * f[qq] + u.x, oacc[qq][dt][1] * f[qq] + u.y,
                        oacc[qq][dt][2] * f[qq] + u.z, oacc[qq][dt][3] * f[qq] + u.w);
      }
  }
  __syncthreads();
  // thread -> (query qi, dims 4 d4 .. +4) for 1024 / NT (query, d4) pairs; the NH wave
  // pair sums added in order
  const int64_t grp = ((int64_t)b * Hq + hq) * nqt + qt;
  constexpr int PAIRS = 1024 / NT;
  float4 acc[PAIRS];
  float Mq[PAIRS], Lq[PAIRS];
#pragma unroll
  for (int it = 0; it < PAIRS; ++it) {
    const int e = threadIdx.x + NT * it;
    const int qi = e >> 5, d4 = (e & 31) * 4;
    acc[it] = *reinterpret_cast<const float4*>(&osum[0][qi][d4]);
#pragma unroll
    for (int ww = 1; ww < NH; ++ww) {
      const float4 u = *reinterpret_cast<const float4*>(&osum[ww][qi][d4]);
      acc[it].x += u.x; acc[it].y += u.y; acc[it].z += u.z; acc[it].w += u.w;
    }
    float M = red_m[0][qi];
    for (int i = 1; i < NW; ++i) M = fmaxf(M, red_m[i][qi]);
    float L = 0.f;
    for (int i = 0; i < NW; ++i)
      L += (red_m[i][qi] == -INFINITY) ? 0.f : red_l[i][qi] * __builtin_amdgcn_exp2f(red_m[i][qi] - M);
    Mq[it] = M;
    Lq[it] = L;
  }
  auto store_o = [&](int qi, int d4, float4 a, float L) {
    const int row = qt * 32 + qi;
    if (row < R) {
      const float inv = 1.0f / L;
      u16x4 r;
      r[0] = f2bf(a.x * inv); r[1] = f2bf(a.y * inv); r[2] = f2bf(a.z * inv); r[3] = f2bf(a.w * inv);
      *reinterpret_cast<u16x4*>(o + ((int64_t)b * R + row) * (Hq * HD) + hq * HD + d4) = r;
    }
  };
  if (nchunk == 1) {
#pragma unroll
    for (int it = 0; it < PAIRS; ++it) {
      const int e = threadIdx.x + NT * it;
      store_o(e >> 5, (e & 31) * 4, acc[it], Lq[it]);
    }
    return;
  }
  float* pc = part + (grp * nchunk + chunk) * kPartStride;
#pragma unroll
  for (int it = 0; it < PAIRS; ++it) {
    const int e = threadIdx.x + NT * it;
    const int qi = e >> 5, d4 = (e & 31) * 4;
    part_store_o(pc, qi, d4, acc[it].x, acc[it].y, acc[it].z, acc[it].w);
    if (d4 == 0) {
      pc[kPartML + qi] = Mq[it];
      pc[kPartML + 32 + qi] = Lq[it];
    }
  }
}

// ============================================================================
// Split-KV attention with one 32-key sub-tile per wave and the P.V product split over the
// head dim: grid (Hq*nqt, nchunk, B), NW waves, chunks of NW*32 keys, 32 query rows.
// Wave w scores sub-tile w (S^T = K . Q^T as in attn_splitkv_bf16); the waves exchange
// their row maxima, so every P is taken against the chunk maximum M, and hand P over
// through LDS as bf16 (2 KB per wave); wave w then forms O^T for dims
// [16 DT w, 16 DT (w + 1)) over all NW sub-tiles (DT = 8 / NW 16-dim tiles), reading
// those dims' Vt rows of the whole chunk (1 KB contiguous per sub-tile and 16-dim tile).
// No wave holds a whole 32 x 128 O tile, so no fp32 O goes through LDS: the chunk
// result (O, M, l), or with a single chunk the normalised output, leaves straight from
// each wave's accumulators.  Same products and MFMA count as the per-wave online form.
// ============================================================================
template <int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_splitkv_ds_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, uint16_t* __restrict__ o, int Hq, int Hkv, int R, int S,
    int Sp, int nqt, int nchunk, float scale_log2, float* __restrict__ part) {
  constexpr int NT = NW * 64, DT = 8 / NW;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  __shared__ float red_m[NW][32], red_l[NW][32];
  __shared__ __attribute__((aligned(16))) uint16_t qs[32 * QS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t ps[NW][32][32];  // P [sub-tile][query][key]
  const int chunk = blockIdx.y;
  const int hq = blockIdx.x / nqt, qt = blockIdx.x % nqt, b = blockIdx.z;
  const int hkv = hq / (Hq / Hkv);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, li = l & 15, j = l >> 4;
  const int ckey0 = chunk * NW * 32;  // the chunk's first key
  const int wkey0 = ckey0 + 32 * w;   // this wave's score sub-tile

  // Q tile: read once per workgroup, staged in LDS (rows >= R clamped: never stored)
  constexpr int QP = 512 / NT;
  const uint16_t* qh = q + ((int64_t)b * Hq + hq) * R * HD;
  u32x4 qg[QP];
#pragma unroll
  for (int u = 0; u < QP; ++u) {
    const int e = threadIdx.x + NT * u;
    qg[u] = *reinterpret_cast<const u32x4*>(qh + (int64_t)min(qt * 32 + (e >> 4), R - 1) * HD +
                                            8 * (e & 15));
  }
  const uint16_t* kbase = k + ((int64_t)b * Hkv + hkv) * Sp * HD;
  const uint16_t* vbase = vt + ((int64_t)b * Hkv + hkv) * HD * Sp;
  // K rows of the wave's sub-tile, in the score-row order of attn_splitkv_bf16 (keys >= S
  // read key S - 1: their scores are masked)
  u32x4 kk[2][4];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const int key = min(wkey0 + 8 * (li >> 2) + 4 * tau + (li & 3), S - 1);
    const uint16_t* kp = kbase + (int64_t)key * HD + 8 * j;
#pragma unroll
    for (int st = 0; st < 4; ++st) kk[tau][st] = *reinterpret_cast<const u32x4*>(kp + 32 * st);
  }
  // Vt rows of the wave's dims for every sub-tile: dim 16 (DT w + dt) + li, keys
  // 32 s + 8j .. +8 of the chunk (masked where used, on sub-tiles that reach S)
  u32x4 vv[NW][DT];
#pragma unroll
  for (int s = 0; s < NW; ++s)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      vv[s][dt] = load8_raw(vbase, 16 * (DT * w + dt) + li, ckey0 + 32 * s + 8 * j, Sp);
#pragma unroll
  for (int u = 0; u < QP; ++u) {
    const int e = threadIdx.x + NT * u;
    *reinterpret_cast<u32x4*>(&qs[(e >> 4) * QS_LD + 8 * (e & 15)]) = qg[u];
  }
  __syncthreads();

  // scores of the wave's 32 keys for both 16-query tiles: lane holds keys wkey0 + 8j + e
  float p[2][8];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    u32x4 qf[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
      qf[st] = *reinterpret_cast<const u32x4*>(&qs[(16 * qq + li) * QS_LD + 8 * j + 32 * st]);
    f32x4 sc[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      sc[tau] = f32x4{};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        sc[tau] = mfma16(as_bf16x8(kk[tau][st]), as_bf16x8(qf[st]), sc[tau]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (wkey0 + 8 * j + e < S) ? sc[e >> 2][e & 3] * scale_log2 : -INFINITY;
      p[qq][e] = x;
      mx = fmaxf(mx, x);
    }
    mx = xor32_combine(xor16_combine(mx, fmax_op), fmax_op);
    if (j == 0) red_m[w][16 * qq + li] = mx;
  }
  __syncthreads();
  // P against the chunk maximum (a row with no valid key in the chunk gets P = 0, l = 0)
  float M[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int qi = 16 * qq + li;
    float m = red_m[0][qi];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = fmaxf(m, red_m[i][qi]);
    M[qq] = m;
    float ls = 0.f;
    u16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(p[qq][e] - m);
      ls += x;
      pb[e] = f2bf(x);
    }
    ls = xor32_combine(xor16_combine(ls, add_op), add_op);
    if (j == 0) red_l[w][qi] = ls;
    *reinterpret_cast<u16x8*>(&ps[w][qi][8 * j]) = pb;
  }
  __syncthreads();

  // O^T (dims x queries) += Vt . P^T over the chunk's sub-tiles
  f32x4 oacc[2][DT];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[qq][dt] = f32x4{};
#pragma unroll
  for (int s = 0; s < NW; ++s) {
    const int key0 = ckey0 + 32 * s;
    const bool tail = key0 + 32 > S;  // uniform over the workgroup
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const bf16x8 pop = as_bf16x8(*reinterpret_cast<const u32x4*>(&ps[s][16 * qq + li][8 * j]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x4 va = tail ? mask8(vv[s][dt], S - (key0 + 8 * j)) : vv[s][dt];
        oacc[qq][dt] = mfma16(as_bf16x8(va), pop, oacc[qq][dt]);
      }
    }
  }
  // lane holds dims 16 (DT w + dt) + 4j + r of query 16 qq + li
  float L[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) s += red_l[i][16 * qq + li];
    L[qq] = s;
  }
  if (nchunk == 1) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int row = qt * 32 + 16 * qq + li;
      if (row < R) {
        const float inv = 1.0f / L[qq];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f32x4 a = oacc[qq][dt];
          *reinterpret_cast<u16x4*>(o + ((int64_t)b * R + row) * (Hq * HD) + hq * HD +
                                    16 * (DT * w + dt) + 4 * j) =
              u16x4{f2bf(a[0] * inv), f2bf(a[1] * inv), f2bf(a[2] * inv), f2bf(a[3] * inv)};
        }
      }
    }
    return;
  }
  const int64_t grp = ((int64_t)b * Hq + hq) * nqt + qt;
  float* pc = part + (grp * nchunk + chunk) * kPartStride;
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int qi = 16 * qq + li;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 a = oacc[qq][dt];
      part_store_o(pc, qi, 16 * (DT * w + dt) + 4 * j, a[0], a[1], a[2], a[3]);
    }
    if (w == 0 && j == 0) {
      pc[kPartML + qi] = M[qq];
      pc[kPartML + 32 + qi] = L[qq];
    }
  }
}

// ============================================================================
// Grouped-query step attention (G = Hq / Hkv query heads per KV head, 2 <= G <= 8, at
// most 32 query rows): grid (B * Hkv, nchunk), 8 waves.  Wave w < G takes query head
// hkv * G + w through every 32-key sub-tile of the chunk; the chunk's K and Vt are read
// from memory once per KV head into LDS (direct global->LDS loads) instead of once per
// query head, and each wave reads them from there in the split-KV kernel's operand
// layout.  Each wave writes its head's chunk result (O, m, l) in attn_combine's layout,
// or, with a single chunk, the normalised output.
//   LDS per 32-key sub-tile: K [32 keys][256 B] with 16-byte chunk c of key r at
//   c ^ ((r % 4) + 4 (r / 8)), then Vt [128 dims][64 B] with chunk c of dim d at
//   c ^ ((d / 4) % 4): the operand reads (16 rows at one chunk per LDS clock) are then
//   conflict free.
// ============================================================================
constexpr int GQ_SUB = 16 * 1024;   // LDS bytes per 32-key sub-tile (K 8 KB, Vt 8 KB)
constexpr int GQ_MAXSUB = 8;        // at most 256 keys per chunk (128 KB of LDS)

__device__ __forceinline__ int gq_kswz(int r) { return (r & 3) | ((r >> 3) << 2); }

// NSUB: the chunk's 32-key sub-tiles, a compile-time count so that the walk over a full
// chunk is unrolled and the scheduler can start a sub-tile's operand reads and score
// products while the previous one is in its softmax.
template <int NSUB>
__global__ __launch_bounds__(512, 1) void attn_gqa_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vt, uint16_t* __restrict__ o, int Hq, int Hkv, int R, int S,
    int Sp, int nchunk, float scale_log2, float* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) unsigned char gsm[];
  constexpr int ck = 32 * NSUB;
  const int chunk = blockIdx.y, b = blockIdx.x / Hkv, hkv = blockIdx.x % Hkv;
  const int G = Hq / Hkv;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, li = l & 15, j = l >> 4;
  const int key_lo = chunk * ck;
  const int nsub = (min(ck, S - key_lo) + 31) / 32;  // sub-tiles with a key below S

  // Q^T operands of this wave's head: query 16 qq + li, dims 32 st + 8j .. +8 (rows >= R
  // clamped: computed, never stored; waves w >= G load head G - 1 and stay idle)
  const int hq = hkv * G + min(w, G - 1);
  const uint16_t* qh = q + ((int64_t)b * Hq + hq) * R * HD;
  u32x4 qf[2][4];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int st = 0; st < 4; ++st)
      qf[qq][st] = *reinterpret_cast<const u32x4*>(qh + (int64_t)min(16 * qq + li, R - 1) * HD +
                                                   32 * st + 8 * j);

  // the chunk's K and Vt: 16 loads of 1 KB per sub-tile (8 of K: 4 keys each; 8 of Vt: 16
  // dims each), dealt to the waves in turn; keys past S read key S - 1 (masked scores),
  // Vt chunks past Sp the last valid chunk (masked values)
  const uint16_t* kb = k + ((int64_t)b * Hkv + hkv) * Sp * HD;
  const uint16_t* vb = vt + ((int64_t)b * Hkv + hkv) * HD * Sp;
  for (int i = w; i < nsub * 16; i += 8) {
    const int sub = i >> 4, pc = i & 15;
    unsigned char* base = gsm + sub * GQ_SUB;
    const int key0 = key_lo + 32 * sub;
    const uint16_t* src;
    unsigned char* dst;
    if (pc < 8) {
      const int r = 4 * pc + (l >> 4), c = (l & 15) ^ gq_kswz(r);
      src = kb + (int64_t)min(key0 + r, S - 1) * HD + 8 * c;
      dst = base + pc * 1024;
    } else {
      const int d = 16 * (pc - 8) + (l >> 2), c = (l & 3) ^ ((d >> 2) & 3);
      src = vb + vt_off(d, min(key0 + 8 * c, Sp - 8), HD);
      dst = base + 8192 + (pc - 8) * 1024;
    }
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt((0 & 15) | ((0 >> 4) << 14) | (7 << 4) | (15 << 8));  // vmcnt(0)
  asm volatile("" ::: "memory");
  __syncthreads();
  if (w >= G) return;  // no barrier follows

  f32x4 oacc[2][8];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[qq][dt] = f32x4{};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  auto walk = [&](int sub) {
    const unsigned char* base = gsm + sub * GQ_SUB;
    KVTile16 t;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int r = 8 * (li >> 2) + 4 * tau + (li & 3);
#pragma unroll
      for (int st = 0; st < 4; ++st)
        t.k[tau][st] = *reinterpret_cast<const u32x4*>(
            base + r * (HD * 2) + (((4 * st + j) ^ gq_kswz(r)) * 16));
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + li;
      t.v[dt] = *reinterpret_cast<const u32x4*>(base + 8192 + d * 64 + ((j ^ ((d >> 2) & 3)) * 16));
    }
    consume_subtile(t, key_lo + 32 * sub, qf, oacc, m_run, l_run, S, scale_log2, j);
  };
  if (NSUB <= 4 && nsub == NSUB) {  // a full chunk (all but a ragged last one); longer
                                    // unrolled walks spill
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) walk(sub);
  } else {
    for (int sub = 0; sub < nsub; ++sub) walk(sub);
  }

  // lane holds query 16 qq + li, dims 16 dt + 4j .. +4
  if (nchunk == 1) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int row = 16 * qq + li;
      if (row >= R) continue;
      const float inv = 1.0f / l_run[qq];
      uint16_t* orow = o + ((int64_t)b * R + row) * (Hq * HD) + hq * HD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        u16x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = f2bf(oacc[qq][dt][e] * inv);
        *reinterpret_cast<u16x4*>(orow + 16 * dt + 4 * j) = r;
      }
    }
    return;
  }
  float* pcb = part + ((int64_t)(b * Hq + hq) * nchunk + chunk) * kPartStride;
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int qi = 16 * qq + li;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      part_store_o(pcb, qi, 16 * dt + 4 * j, oacc[qq][dt][0], oacc[qq][dt][1],
                   oacc[qq][dt][2], oacc[qq][dt][3]);
    if (j == 0) {
      pcb[kPartML + qi] = m_run[qq];
      pcb[kPartML + 32 + qi] = l_run[qq];
    }
  }
}

// Merge the chunk partials: o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c, chunks in
// order.  grid (B*Hq*nqt, 8), 128 threads: workgroup y handles query rows 4y .. 4y+3 of
// the 32-row tile, thread -> (row, 4 dims).  Every thread computes its row's weights
// itself (the (m, l) pairs are 2 * nchunk broadcast loads), and the partial loads of up
// to 16 chunks are issued together.
constexpr int kCombRows = 4;
__global__ __launch_bounds__(128) void attn_combine(const float* __restrict__ part,
                                                    uint16_t* __restrict__ o, int Hq, int R,
                                                    int nqt, int nchunk) {
  const int64_t grp = blockIdx.x;
  const int qt = (int)(grp % nqt);
  const int hq = (int)((grp / nqt) % Hq);
  const int b = (int)(grp / ((int64_t)nqt * Hq));
  const int qi = blockIdx.y * kCombRows + (threadIdx.x >> 5), d4 = (threadIdx.x & 31) * 4;
  const int row = qt * 32 + qi;
  const float* pg = part + grp * nchunk * kPartStride;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float M = -INFINITY, L = 0.f;
  for (int c0 = 0; c0 < nchunk; c0 += 16) {
    float mc[16], lc[16];
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int c = min(c0 + u, nchunk - 1);  // clamped; chunks past nchunk are dropped
      const float* pc = pg + (int64_t)c * kPartStride;
      mc[u] = pc[kPartML + qi];
      lc[u] = pc[kPartML + 32 + qi];
      const u16x4 r = *reinterpret_cast<const u16x4*>(reinterpret_cast<const uint16_t*>(pc) +
                                                      qi * HD + d4);
      v[u] = make_float4(bf2f(r[0]), bf2f(r[1]), bf2f(r[2]), bf2f(r[3]));
    }
    // online merge in chunk order (the same result as rescaling by the global max)
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (c0 + u >= nchunk || mc[u] == -INFINITY) continue;
      const float Mn = fmaxf(M, mc[u]);
      const float fa = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      const float fb = __builtin_amdgcn_exp2f(mc[u] - Mn);
      L = L * fa + lc[u] * fb;
      acc.x = acc.x * fa + v[u].x * fb; acc.y = acc.y * fa + v[u].y * fb;
      acc.z = acc.z * fa + v[u].z * fb; acc.w = acc.w * fa + v[u].w * fb;
      M = Mn;
    }
  }
  if (row < R) {
    const float inv = 1.0f / L;
    u16x4 r;
    r[0] = f2bf(acc.x * inv); r[1] = f2bf(acc.y * inv); r[2] = f2bf(acc.z * inv); r[3] = f2bf(acc.w * inv);
    // written through (device-coherent store): the output projection that follows stages
    // it from every XCD (8B cached step about 1 % faster together with the value-cache
    // stores of the QKV reduction)
    st_dev(o + ((int64_t)b * R + row) * (Hq * HD) + hq * HD + d4, r);
  }
}

// ============================================================================
// Flash attention over all rows (refresh, or steps with more than 256 rows):
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

  // K and Vt tiles of the next 64 keys are loaded into registers while the current
  // tile is computed (branch-free: K rows past S read row S-1, whose scores are masked;
  // Vt keys past S read as zero)
  const int ntile = (S + FK - 1) / FK;
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int kt) {
    const int kbase = kt * FK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int r = e >> 4, c8 = e & 15;  // K: 64 rows x 16 chunks
      kreg[i] = *reinterpret_cast<const u32x4*>(kb + (int64_t)min(kbase + r, S - 1) * HD + 8 * c8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int r = e >> 3, c8 = e & 7;   // Vt: 128 rows x 8 chunks of 8 keys
      vreg[i] = load8_raw(vb, r, kbase + 8 * c8, Sp);
    }
  };
  load_tile(0);
  for (int kt = 0; kt < ntile; ++kt) {
    const int kbase = kt * FK;
    __syncthreads();  // every wave is done with the previous tile
    const bool tail = kbase + FK > S;  // uniform: the Vt keys >= S are zeroed
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x + 256 * i;
      *reinterpret_cast<u32x4*>(&Ks[(e >> 4) * KS_LD + 8 * (e & 15)]) = kreg[i];
      *reinterpret_cast<u32x4*>(&Vs[(e >> 3) * VS_LD + 8 * (e & 7)]) =
          tail ? mask8(vreg[i], S - (kbase + 8 * (e & 7))) : vreg[i];
    }
    __syncthreads();
    load_tile(kt + 1);  // past the last tile: clamped addresses, never stored (no branch)
    // keep the prefetch here, ahead of this tile's products (the scheduler would otherwise
    // sink it below them to shorten the registers' live ranges)
    __builtin_amdgcn_sched_barrier(0);

    // raw scores; keys >= S (only in the last tile: a uniform test) count as -inf
    const bool full = kbase + FK <= S;
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
      if (full) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          p[st][v] = s[v];
          tmax = fmaxf(tmax, s[v]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float x = (kbase + st * 32 + acc_row(v, g) < S) ? s[v] : -INFINITY;
          p[st][v] = x;
          tmax = fmaxf(tmax, x);
        }
      }
    }
    // the scale is positive, so the scaled maximum is the maximum of the scaled scores;
    // exp2(score * scale - max) is one FMA per score
    tmax = xor32_combine(tmax, fmax_op) * scale_log2;
    const float m_new = fmaxf(m_run, tmax);   // finite: every tile has a valid key
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float ls = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[st][v] = __builtin_amdgcn_exp2f(fmaf(p[st][v], scale_log2, -m_new));
        ls += p[st][v];
      }
    ls = xor32_combine(ls, add_op);
    l_run = l_run * alpha + ls;
    m_run = m_new;
    // alpha is exactly 1 where the running maximum did not move: rescale only if some
    // lane's did (a uniform branch)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
    }
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
    for (int j = 0; j < S; ++j) a += sc[j] * vb[vt_off(d, j, D)];
    o[((int64_t)b * R + row) * (Hq * D) + hq * D + d] = a / sum;
  }
}

constexpr int kMaxChunks = 64;

// Step attention (at most 256 query rows: a block step, or the block and suffix rows of a
// prefix-mode step, where the 128-row flash tiles would give only 32-64 workgroups; prefix
// workload 926 -> 920 ms per generation), 32-row query tiles, 32-key sub-tiles per wave:
// (plans with one sub-tile per wave run attn_splitkv_ds_bf16: 8B cached step 4.159 ->
// 4.090 ms against the per-wave online form with an LDS merge of the waves' O tiles):
//  * one sub-tile per wave in eight-wave workgroups (256-key chunks: half the partials
//    to merge of four-wave chunks) when that gives 160 to 1024 workgroups (32 query rows
//    x 32 heads against 1032-1500 keys, kernel-only: 14.4-15.7 us with 9-12 four-wave
//    chunks per head, 13.9-14.3 with 5-6 eight-wave ones; with 4 eight-wave chunks, 128
//    workgroups, 1024 keys took 13.4 against 13.0 us);
//  * else one sub-tile per wave in four-wave workgroups if that needs at most 512;
//  * else four waves walking several sub-tiles each (a register-heavy kernel, one
//    workgroup per CU), with chunks sized for about 256 workgroups.
// Keys per chunk of the grouped-query kernel (a multiple of 32, at most 256 for its LDS),
// chosen for about 256 workgroups of B * Hkv * chunks: every wave walks all sub-tiles of
// its chunk, so shorter chunks and more workgroups (7B batch-8 step: 6.88 -> 6.75 ms with
// 128-key chunks against 256); 0 where the kernel does not apply (more than 32 rows or
// another head dim).
static int gqa_chunk_keys(int B, int Hkv, int R, int S, int D) {
  if (R > 32 || D != HD || B * Hkv < 1) return 0;
  const int nchunk = (256 + B * Hkv - 1) / (B * Hkv);
  const int ck = 32 * ((S + 32 * nchunk - 1) / (32 * nchunk));
  return std::min(std::max(ck, 32), 32 * GQ_MAXSUB);
}

AttnPlan attn_plan(int dtype, int B, int Hq, int Hkv, int R, int S, int D) {
  AttnPlan p;
  if (dtype == F32) { p.kind = 0; return p; }
  if (R <= 256) {
    p.kind = 1;
    p.nqt = (R + 31) / 32;
    const int64_t base = (int64_t)B * Hq * p.nqt;
    const int n8 = (S + 255) / 256, n4 = (S + 127) / 128;
    if (base * n8 >= 160 && base * n8 <= 1024 && n8 <= kMaxChunks) {
      p.nw = 8; p.nsub = 1; p.nchunk = n8;
    } else if (base * n4 <= 512 && n4 <= kMaxChunks) {
      p.nw = 4; p.nsub = 1; p.nchunk = n4;
    } else {
      int64_t target = (256 + base - 1) / base;      // chunks wanted for ~256 workgroups
      if (target < 1) target = 1;
      int ck = (int)((S + target - 1) / target);     // keys per chunk
      ck = (ck + 127) / 128 * 128;                   // 4 waves x 32-key sub-tiles
      if ((S + ck - 1) / ck > kMaxChunks) ck = ((S + kMaxChunks - 1) / kMaxChunks + 127) / 128 * 128;
      p.nw = 4; p.nsub = ck / 128; p.nchunk = (S + ck - 1) / ck;
    }
    if (p.nchunk > 1) p.part_floats = (size_t)base * p.nchunk * kPartStride;
    // grouped query heads: each chunk's K and Vt read once per KV head
    const int G = (Hkv > 0 && Hq % Hkv == 0) ? Hq / Hkv : 1;
    const int ck = (G >= 2 && G <= 8) ? gqa_chunk_keys(B, Hkv, R, S, D) : 0;
    if (ck > 0) {
      p.kind = 3;
      p.ck = ck;
      p.nchunk = (S + ck - 1) / ck;
      p.part_floats = p.nchunk > 1 ? (size_t)base * p.nchunk * kPartStride : 0;
    }
  } else {
    p.kind = 2;
    p.nqt = (R + 127) / 128;
  }
  return p;
}

size_t attn_part_floats_any_hkv(int dtype, int B, int Hq, int R, int S, int D) {
  size_t n = attn_plan(dtype, B, Hq, Hq, R, S, D).part_floats;
  for (int G = 2; G <= 8; ++G)
    if (Hq % G == 0) n = std::max(n, attn_plan(dtype, B, Hq, Hq / G, R, S, D).part_floats);
  return n;
}

hipError_t launch_attention(int dtype, const AttnPlan& p, const void* q, const void* k,
                            const void* vt, void* o, int B, int Hq, int Hkv, int R, int S, int Sp,
                            int D, float* part, int* counters, hipStream_t st) {
  (void)counters;
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
    if (p.nchunk > 1 && !part) return hipErrorInvalidValue;
    // one sub-tile per wave: head-major, workgroup ids running over (head, query tile)
    // first, so with Hq * nqt a multiple of 8 every chunk of one head lands on one XCD
    // and the head's Q tile is read from memory once per XCD rather than once per chunk
    // (8B cached step 4.085 -> 4.064 ms, bit-identical); several sub-tiles per wave (long
    // key ranges, where the Q tile is a small share of a chunk's bytes): chunk-major
    // (16384 keys kernel-only 60.5 -> 59.6 us against head-major)
    const dim3 grid(Hq * p.nqt, p.nchunk, B);
#define DLLM_ATTN(NWV)                                                                        \
  attn_splitkv_bf16<NWV><<<dim3(p.nchunk, Hq * p.nqt, B), NWV * 64, 0, st>>>(                 \
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)vt, (uint16_t*)o, Hq, Hkv, R, S, \
      Sp, p.nqt, p.nchunk, p.nsub, scale_log2, part)
#define DLLM_ATTN_DS(NWV)                                                                     \
  attn_splitkv_ds_bf16<NWV><<<grid, NWV * 64, 0, st>>>(                                       \
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)vt, (uint16_t*)o, Hq, Hkv, R, S, \
      Sp, p.nqt, p.nchunk, scale_log2, part)
    if (p.nw == 8 && p.nsub == 1) DLLM_ATTN_DS(8);
    else if (p.nw == 4 && p.nsub == 1) DLLM_ATTN_DS(4);
    else if (p.nw == 4) DLLM_ATTN(4);
    else return hipErrorInvalidValue;  // the plan never asks for 8 waves x several sub-tiles
#undef DLLM_ATTN
#undef DLLM_ATTN_DS
    if (p.nchunk > 1) {
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      attn_combine<<<dim3((unsigned)(B * Hq * p.nqt), 32 / kCombRows), 32 * kCombRows, 0, st>>>(
          part, (uint16_t*)o, Hq, R, p.nqt, p.nchunk);
    }
  } else if (p.kind == 3) {
    if (p.nchunk > 1 && !part) return hipErrorInvalidValue;
    static bool attr_set[GQ_MAXSUB + 1] = {};  // opt in to > 64 KB of dynamic LDS once each
    const int nsubk = p.ck / 32;
    if (p.ck % 32 != 0 || nsubk < 1 || nsubk > GQ_MAXSUB) return hipErrorInvalidValue;
#define DLLM_GQA(NS)                                                                          \
  do {                                                                                        \
    if (!attr_set[NS]) {                                                                      \
      hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_gqa_bf16<NS>), \
                                           hipFuncAttributeMaxDynamicSharedMemorySize,        \
                                           NS * GQ_SUB);                                      \
      if (err != hipSuccess) return err;                                                      \
      attr_set[NS] = true;                                                                    \
    }                                                                                         \
    attn_gqa_bf16<NS><<<dim3(B * Hkv, p.nchunk), 512, NS * GQ_SUB, st>>>(                     \
        (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)vt, (uint16_t*)o, Hq, Hkv, R, \
        S, Sp, p.nchunk, scale_log2, part);                                                   \
  } while (0)
    switch (nsubk) {
      case 1: DLLM_GQA(1); break;
      case 2: DLLM_GQA(2); break;
      case 3: DLLM_GQA(3); break;
      case 4: DLLM_GQA(4); break;
      case 5: DLLM_GQA(5); break;
      case 6: DLLM_GQA(6); break;
      case 7: DLLM_GQA(7); break;
      default: DLLM_GQA(8); break;
    }
#undef DLLM_GQA
    if (p.nchunk > 1) {
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      attn_combine<<<dim3((unsigned)(B * Hq * p.nqt), 32 / kCombRows), 32 * kCombRows, 0, st>>>(
          part, (uint16_t*)o, Hq, R, p.nqt, p.nchunk);
    }
  } else {
    attn_flash_bf16<<<dim3(p.nqt, Hq, B), 256, 0, st>>>(
        (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)vt, (uint16_t*)o, Hq, Hkv, R,
        S, Sp, scale_log2);
  }
  return hipGetLastError();
}

}  // namespace dllm
