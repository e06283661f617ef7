// decode.hip -- split-K single-token decode attention over the packed cache (all three
// formats, any supported GQA group), plus the log-sum-exp merge of the splits.
//
// Semantics: bxzpzcl.cn/news/2871434 section 3.2 (window [len - W, len), query head h
// reads KV head h / (Hq / Hkv), softmax scale head_dim^-1/2); lpnh.cn/news/2042373
// section 1.1 (each decode step attends over the whole cache); the operator reads the
// packed data and dequantizes inside ("LLM长上下文推理优化：用INT4状态机管理KV Cache",
// pwwt.cn/news/4219524, section 5 step 5).
//
// Stage 1 (decode_splitk_kernel): one workgroup per (split, kv head, batch).  A row of
// D values spans D/8 lanes (8 values per lane), so a 256-lane workgroup walks 2048/D
// positions at a time, 4 per lane group per step with the next step's rows already in
// flight; the G query heads of the KV head share every K/V load.  Scores are kept in
// log2 units (q is pre-scaled by scale * log2 e) with an online softmax per lane row;
// the rows are combined through LDS and the workgroup writes one unnormalized partial
// (max, sum, weighted V) per query head.
// Stage 2: out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i, inside stage 1 by the
// last split of a (b, kv head) when there are at most 32 splits, otherwise by
// merge_kernel (one workgroup per query head).
// Codec: keys/values stay in the rotated domain.  Since H/sqrt(D) is orthonormal and
// symmetric, q . x_hat = (H q / sqrt(D)) . (s c[idx]); q is rotated once per workgroup
// and the merged output is rotated back once per (b, h).  With the append fused, the
// last split codes the new row (the same row encoder as the append kernel) and attends
// it from registers.
#include <cmath>

#include "kvq_arith.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float NEG_INF = -__builtin_huge_valf();

// Device-scope (every XCD) store / loads of the split partials, for the in-kernel merge.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// an 8-byte-aligned (max, sum) pair in one load
__device__ __forceinline__ uint64_t fetch_pair(const float* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// The packed bytes lane c owns of one row (cache row index b*Hkv*C + slot): its code
// word(s) and the scale of its group, for K and V.  Loaded for several rows before any
// of them is used, so that a lane keeps several rows' transfers in flight.
struct RawRow {
  uint32_t k[2], v[2];   // INT4 / codec: k[0], v[0] (8 nibbles); INT8: both (8 bytes)
  float sk, sv;
};

template <int D, int FMT>
__device__ __forceinline__ RawRow load_raw(const DecodeArgs& a, size_t row, int c) {
  constexpr int LPR = D / 8;
  RawRow r;
  if (FMT == KVQ_INT8_TOKEN) {
    const uint2 kw = reinterpret_cast<const uint2*>(a.k_codes)[row * LPR + c];
    const uint2 vw = reinterpret_cast<const uint2*>(a.v_codes)[row * LPR + c];
    r.k[0] = kw.x; r.k[1] = kw.y; r.v[0] = vw.x; r.v[1] = vw.y;
    r.sk = a.k_scales[row];
    r.sv = a.v_scales[row];
  } else if (FMT == KVQ_WHT_LM3) {   // one aligned dword of the packed row per lane
    // (its 24 bits are assembled where the row is used: packed3_bits)
    r.k[0] = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.k_codes) + row * 3 * LPR)[packed3_dword(c)];
    r.v[0] = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.v_codes) + row * 3 * LPR)[packed3_dword(c)];
    r.k[1] = r.v[1] = 0u;
    r.sk = a.k_scales[row];
    r.sv = a.v_scales[row];
  } else {
    r.k[0] = reinterpret_cast<const uint32_t*>(a.k_codes)[row * LPR + c];
    r.v[0] = reinterpret_cast<const uint32_t*>(a.v_codes)[row * LPR + c];
    r.k[1] = r.v[1] = 0u;
    if (FMT == KVQ_INT4_G) {
      r.sk = a.k_scales[row * (D / a.gk) + (8 * c) / a.gk];
      r.sv = a.v_scales[row * (D / a.gv) + (8 * c) / a.gv];
    } else if (FMT == KVQ_INT4_G16) {   // fp16 scales
      r.sk = (float)reinterpret_cast<const _Float16*>(a.k_scales)[row * (D / a.gk) + (8 * c) / a.gk];
      r.sv = (float)reinterpret_cast<const _Float16*>(a.v_scales)[row * (D / a.gv) + (8 * c) / a.gv];
    } else {
      r.sk = a.k_scales[row];
      r.sv = a.v_scales[row];
    }
  }
  return r;
}

// The 8 code values of a code word pair as floats, before the scale (integers for INT4
// and INT8, codebook levels for the codec).  A lane's 8 values share one scale (groups
// are powers of two of at least 32), which is applied once per dot product instead.
template <int FMT>
__device__ __forceinline__ void codes_f32(const uint32_t w[2], const float2* lv2, float x[8]) {
  if (FMT == KVQ_INT4_G || FMT == KVQ_INT4_G16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (float)nib_s(w[0], j);
  } else if (FMT == KVQ_INT8_TOKEN) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = (float)(int8_t)((w[0] >> (8 * j)) & 255u);
      x[j + 4] = (float)(int8_t)((w[1] >> (8 * j)) & 255u);
    }
  } else if (FMT == KVQ_WHT_LM3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // w[0]: the lane's 24 bits; one lookup per index pair
      const float2 p = lv2[(w[0] >> (6 * i)) & 63u];
      x[2 * i] = p.x;
      x[2 * i + 1] = p.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // one lookup per byte: its two levels (low nibble first)
      const float2 p = lv2[(w[0] >> (8 * i)) & 255u];
      x[2 * i] = p.x;
      x[2 * i + 1] = p.y;
    }
  }
}

// Up to this many splits, the last split of a (sequence, KV head) merges the partials
// inside the split-K kernel; above, the merge kernel does.  (64 measured slower on the
// Gemma step's 64-split layers: every split then waits for its stores' acknowledgement
// and for an arrival counter that 64 workgroups update one after another, where
// otherwise they store and exit.)
constexpr int MERGE_INLINE_MAX = 32;

// Threads per workgroup: 512 for the codecs at D = 256 (16 row groups of 32 lanes: a
// split of 128 rows is two row steps, and half as many splits write and merge partials
// as with 256 threads and 64-row splits), 256 otherwise.
__host__ __device__ constexpr int splitk_threads(int D, int FMT) {
  return (FMT == KVQ_WHT_LM4 || FMT == KVQ_WHT_LM3) && D == 256 ? 512 : 256;
}

template <int D, int G, int FMT>
__global__ void __launch_bounds__(splitk_threads(D, FMT)) decode_splitk_kernel(DecodeArgs a) {
  constexpr bool CODEC = FMT == KVQ_WHT_LM4 || FMT == KVQ_WHT_LM3;
  constexpr int NT = splitk_threads(D, FMT);
  constexpr int NW = NT / 64;   // waves
  constexpr int LPR = D / 8;
  constexpr int NGRP = NT / LPR;
  __shared__ float s_m[NGRP][G];
  __shared__ float s_l[NGRP][G];
  __shared__ float s_acc[NGRP][G][D];
  __shared__ float2 lv2[CODEC ? 256 : 1];   // codec: the levels of a byte's nibbles
  // codec: q rotated and scaled, [G][D] (read and written as float4)
  __shared__ __attribute__((aligned(16))) float s_q[CODEC ? G * D : 1];

  const int sp = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, grp = tid / LPR, c = tid % LPR;
  // q first: its load heads the critical path.  The codec rotates q once per workgroup:
  // row group NGRP - G + h (the last ones, which never code the fused append's row)
  // loads, rotates and scales head h and stages it in LDS; every thread reads its dims
  // of each head after the barrier below.  (Rotated by every row group, the transform
  // held every wave for ~0.7 us before the first row.)  Issued here, ahead of the split
  // bounds, the load follows the first read of the argument block; placed after them, it
  // waited for a second one.
  const uint16_t* qb = a.q + (size_t)(b * a.Hq + kvh * G) * D;   // head 0 of this KV head
  uint4 qraw[CODEC ? 1 : G];
  [[maybe_unused]] const int hq = grp - (NGRP - G);   // codec: the head this group rotates
  if constexpr (CODEC) {
    if (hq >= 0) qraw[0] = *reinterpret_cast<const uint4*>(qb + (size_t)hq * D + 8 * c);
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) qraw[h] = *reinterpret_cast<const uint4*>(qb + (size_t)h * D + 8 * c);
  }
  const int len = a.lens[b];
  const int lo = a.window > 0 ? max(0, len - a.window) : 0;
  // codec or INT4 with fp16 scales, with the append fused: position len - 1 is the new
  // row, coded in this kernel and attended from registers by the last split, which
  // (when there are several) has no other rows: the other splits cover [lo, len - 1)
  const bool fused = (CODEC || FMT == KVQ_INT4_G16) && a.k_new != nullptr;
  const bool app_split = fused && sp == a.nsplit - 1;
  const int nrs = fused && a.nsplit > 1 ? a.nsplit - 1 : a.nsplit;   // splits with rows
  const int pt = fused ? len - 1 : len;
  // with a window, the attention sinks [0, nsk) come first: the splits share out the
  // virtual range [vlo, pt), where u in [vlo, lo) stands for position u - vlo
  const int nsk = a.window > 0 ? min(a.sinks, lo) : 0;
  const int vlo = lo - nsk;
  const int span = pt - vlo;
  const int chunk = span > 0 ? (span + nrs - 1) / nrs : 0;
  const int ps = sp < nrs ? min(pt, vlo + sp * chunk) : pt;
  const int pe = min(pt, ps + chunk);

  // the rows of the first two steps are requested before q is rotated, so their
  // latency overlaps it (a split of up to 2 U NGRP rows has all of its rows in
  // flight at once); each later step's rows are requested one step ahead (see the
  // row loop below)
  constexpr int U = 4;
  constexpr int SR = U * NGRP;   // rows per step (all groups)
  const size_t bh = (size_t)b * a.Hkv + kvh;
  auto load_step = [&](int t0, RawRow (&raw)[U]) {
    if (a.pages.size) {   // (uniform) paged layout: each row through the block table
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = min(t0 + u * NGRP, pe - 1);
        raw[u] = load_raw<D, FMT>(a, paged_row(a.pages, a.Hkv, b, kvh, t), c);
      }
    } else if (a.sinks == 0) {   // (uniform) one ring: slot t mod cap
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = min(t0 + u * NGRP, pe - 1);
        raw[u] = load_raw<D, FMT>(a, bh * a.cap + (t % a.cap), c);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = min(t0 + u * NGRP, pe - 1);
        raw[u] = load_raw<D, FMT>(a, bh * a.cap + cache_slot(t >= lo ? t : t - vlo, a.cap, a.sinks), c);
      }
    }
  };
  // then the codebook levels, then the rows
  // codec: this thread's entry of the level table, the two levels of a byte (4 bits) or of
  // a 6-bit index pair (3 bits); requested here, the loads overlap q's (requested after
  // q's rotation they were a round trip of their own before the first row step)
  [[maybe_unused]] float2 lvv;
  if (CODEC && tid < 256)
    lvv = FMT == KVQ_WHT_LM3 ? make_float2(a.levels[tid & 7], a.levels[(tid >> 3) & 7])
                             : make_float2(a.levels[tid & 15], a.levels[tid >> 4]);
  int t0 = ps + grp;
  RawRow cur[U], nxt[U];
  if (t0 < pe) load_step(t0, cur);
  if (t0 + SR < pe) load_step(t0 + SR, nxt);
  // the append split: row group 0 codes the new K row and row group 1 the new V row,
  // side by side in wave 0 (fp16 rows requested here and coded as soon as they arrive;
  // wave 0 takes no part in q's rotation); group 0 then attends the new row (after its
  // cached rows, if the split has any)
  const bool app_wave = app_split && tid < 64;   // wave-uniform
  const bool app_grp = app_wave && grp == 0;
  uint4 newx = make_uint4(0u, 0u, 0u, 0u);
  Thresholds thr;
  if (app_wave) {
    if (grp < 2) newx = *reinterpret_cast<const uint4*>((grp ? a.v_new : a.k_new) + bh * D + 8 * c);
    if (CODEC) thr = load_thresholds(a.thr);
  }

  // (the levels arrive with q: stored now, they hold no registers through q's rotation)
  if (CODEC && tid < 256) lv2[tid] = lvv;
  float q[G][8];
  if constexpr (CODEC) {
    if (hq >= 0) {   // (whole row groups: the transform's lane exchanges stay inside)
      float x[8];
      f16x8_unpack(qraw[0], x);
      wht_row<LPR>(x, c);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] *= 1.0f / sqrtf((float)D);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] *= a.qscale;
      *reinterpret_cast<float4*>(s_q + hq * D + 8 * c) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4*>(s_q + hq * D + 8 * c + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      f16x8_unpack(qraw[h], q[h]);
#pragma unroll
      for (int j = 0; j < 8; ++j) q[h][j] *= a.qscale;
    }
  }
  RawRow nr;
  if (app_wave) {
    // coded as the append kernel codes it (every lane of the wave runs the coder, so
    // its lane exchanges stay inside active rows) and written to the row's slot, which
    // no other split reads: it is outside [lo, len - 1) and holds no horizon position
    float x[8];
    f16x8_unpack(newx, x);
    uint32_t w;
    float sc;
    if constexpr (CODEC) {
      codec_encode_row<LPR>(x, c, thr, w, sc);
    } else {   // INT4 with fp16 scales: the quantize kernel's arithmetic, group amax by DPP
      float am = abs_max8(x);
      auto group_max = [](float v, int lanes) {   // (uniform switch)
        switch (lanes) {
          case 4: return lane_group_max<4>(v);
          case 8: return lane_group_max<8>(v);
          case 16: return lane_group_max<16>(v);
          default: return lane_group_max<32>(v);
        }
      };
      const float amk = group_max(am, a.gk >> 3), amv = group_max(am, a.gv >> 3);
      const float s16 = (float)(_Float16)((grp == 1 ? amv : amk) / 7.0f);
      sc = s16 == 0.0f ? 1.0f : s16;
      w = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float y = (float)(_Float16)(x[j] / sc);
        w |= (kvq_round_bits(fminf(fmaxf(y, -7.0f), 7.0f)) & 15u) << (4 * j);
      }
    }
    if (grp < 2) {
      const size_t row = a.pages.size ? paged_row(a.pages, a.Hkv, b, kvh, len - 1)
                                      : bh * a.cap + cache_slot(len - 1, a.cap, a.sinks);
      void* codes = const_cast<void*>(grp ? a.v_codes : a.k_codes);
      if (FMT == KVQ_WHT_LM3) store_packed3<LPR>(static_cast<uint8_t*>(codes) + row * 3 * LPR, c, w);
      else static_cast<uint32_t*>(codes)[row * LPR + c] = w;
      if (FMT == KVQ_INT4_G16) {   // the group's fp16 scale, from its first lane
        const int g = grp ? a.gv : a.gk;
        if ((8 * c) % g == 0)
          reinterpret_cast<_Float16*>(const_cast<float*>(grp ? a.v_scales : a.k_scales))[row * (D / g) + (8 * c) / g] =
              (_Float16)sc;
      } else if (c == 0) {
        const_cast<float*>(grp ? a.v_scales : a.k_scales)[row] = sc;
      }
    }
    // group 0 takes the V row's word and scale from the lane LPR above it (3 bits: the
    // word as the lane's 24 packed bits, the form the row loop looks levels up from)
    if (FMT == KVQ_WHT_LM3) w = packed3_of_nibbles(w);
    const int src = ((tid + LPR) & 63) << 2;
    nr.k[0] = w;
    nr.sk = sc;
    nr.v[0] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)w);
    nr.sv = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, sc)));
    nr.k[1] = nr.v[1] = 0u;
  }

  if constexpr (CODEC) {   // the level table and the rotated q (stored above) are complete
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float4 lo4 = *reinterpret_cast<const float4*>(s_q + h * D + 8 * c);
      const float4 hi4 = *reinterpret_cast<const float4*>(s_q + h * D + 8 * c + 4);
      q[h][0] = lo4.x; q[h][1] = lo4.y; q[h][2] = lo4.z; q[h][3] = lo4.w;
      q[h][4] = hi4.x; q[h][5] = hi4.y; q[h][6] = hi4.z; q[h][7] = hi4.w;
    }
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = NEG_INF;
    l[h] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.0f;
  }

  // U rows per lane group per step.  The step scores its U rows, rescales the
  // accumulators once by 2^(m - m_new) (1 when no head's maximum grew; 0 for the first
  // rows, m being -inf before them: a multiply costs less than the register copies the
  // compiler adds around a conditional rescale), then adds the U rows.  Rows past pe
  // (last step only) are loaded clamped to pe - 1 and scored -inf; they are the same
  // rows for the LPR lanes of a row, and every lane of a row takes part in the row's
  // lane sums.
  // (3 bits: a cached row's words are the lane's aligned dwords of the packed row, whose
  // 24 bits packed3_bits assembles here, where the row is used, so that the row loads
  // stay in flight until then; the fused append's row arrives assembled)
  const int quad = c & 3;
  auto bits_of = [&](const uint32_t (&w)[2], bool assembled, uint32_t (&o)[2]) {
    o[0] = FMT == KVQ_WHT_LM3 && !assembled ? packed3_bits(w[0], quad) : w[0];
    o[1] = w[1];
  };
  auto do_step = [&](const RawRow (&raw)[U], int nvalid, bool assembled = false) {
    float z[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kc[8];
      uint32_t kw[2];
      bits_of(raw[u].k, assembled, kw);
      codes_f32<FMT>(kw, lv2, kc);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) d = __builtin_fmaf(q[h][j], kc[j], d);
        // the lane's partial dot product times its K scale, summed over the row
        const float zz = lane_group_sum<LPR>(d * raw[u].sk);
        z[u][h] = u < nvalid ? zz : NEG_INF;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mn = m[h];
#pragma unroll
      for (int u = 0; u < U; ++u) mn = fmaxf(mn, z[u][h]);
      const float corr = fast_exp2(m[h] - mn);   // (row 0 is valid: mn > -inf)
      l[h] *= corr;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[h][j] *= corr;
      m[h] = mn;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vc[8];
      uint32_t vw[2];
      bits_of(raw[u].v, assembled, vw);
      codes_f32<FMT>(vw, lv2, vc);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = fast_exp2(z[u][h] - m[h]);
        l[h] += p;
        const float pv = p * raw[u].sv;   // the V scale folded into the weight
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = __builtin_fmaf(vc[j], pv, acc[h][j]);
      }
    }
  };
  // the first step (its successor already in flight), then one step per iteration,
  // each requesting the next step's rows before it computes (a loop that carried both
  // buffers across iterations would need more registers)
  if (t0 < pe) {
    do_step(cur, min(U, (pe - t0 + NGRP - 1) / NGRP));
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    t0 += SR;
  }
  while (t0 < pe) {
    const int t1 = t0 + SR;
    if (t1 < pe) load_step(t1, nxt);   // the next step's rows, in flight during this one
    do_step(cur, min(U, (pe - t0 + NGRP - 1) / NGRP));
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    t0 = t1;
  }
  if (app_grp) {   // the new row: one more row of this group's softmax
    const RawRow raw[U] = {nr, nr, nr, nr};
    do_step(raw, 1, true);
  }

  if (c == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[grp][h] = m[h];
      s_l[grp][h] = l[h];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) s_acc[grp][h][8 * c + j] = acc[h][j];
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D, d = idx % D;
    float M = NEG_INF;
#pragma unroll
    for (int gi = 0; gi < NGRP; ++gi) M = fmaxf(M, s_m[gi][h]);
    float A = 0.0f, L = 0.0f;
    if (M != NEG_INF) {   // (a group that saw no row has max -inf: weight 2^-inf = 0)
#pragma unroll
      for (int gi = 0; gi < NGRP; ++gi) {
        const float w = fast_exp2(s_m[gi][h] - M);
        A = __builtin_fmaf(s_acc[gi][h][d], w, A);
        L = __builtin_fmaf(s_l[gi][h], w, L);
      }
    }
    const size_t o = (size_t)(b * a.Hq + kvh * G + h) * a.nsplit + sp;
    if (a.merge_inline) {
      publish(a.ws_acc + o * D + d, A);
      if (d == 0) {
        publish(a.ws_ml + 2 * o, M);
        publish(a.ws_ml + 2 * o + 1, L);
      }
    } else {
      a.ws_acc[o * D + d] = A;
      if (d == 0) {
        a.ws_ml[2 * o] = M;
        a.ws_ml[2 * o + 1] = L;
      }
    }
  }
  if (!a.merge_inline) return;

  // ---- in-kernel merge (few splits): every wave waits for its partial stores, the
  // workgroup counts itself in with a device-scope atomic, and the last split of the
  // (b, kv head) merges the partials with the log-sum-exp rule (the codec's output is
  // rotated back), then resets the counter for the next call.  The order rests on the
  // same hardware properties as the matrix-core kernel's merge (decode_mfma.hip,
  // "arrivals"): acknowledged device-scope stores are visible to device-scope loads on
  // every XCD, increments follow their workgroup's acknowledgements, and the merging
  // workgroup's loads follow its increment's return.
  __shared__ int s_last;
  uint32_t* cnt = a.counters + (size_t)b * a.Hkv + kvh;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) s_last = (int)__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int np = a.nsplit;
  if (s_last != np - 1) return;
  const size_t pbase = (size_t)(b * a.Hq + kvh * G) * np;   // partial of (head 0, split 0)
  static_assert(MERGE_INLINE_MAX <= 64, "one split per lane");
  float* s_w = &s_acc[0][0][0];       // [G][64] split weights (0 past np)
  float* s_L = s_w + G * 64;          // [G] weighted sums of the split sums
  float* s_out = s_L + G;             // [G][D] merged output (codec: before the rotation)
  const int wave = tid >> 6, lane = tid & 63;
  // every thread first requests its outputs' first partials (up to 64 loads), and wave
  // w the (max, sum) pairs of heads w, w + 4, ... (split = lane), so that up to PF
  // splits are one round trip; the partial loads go in groups of 8 under a uniform test,
  // the split index clamped to np - 1 inside a group (their weight is 0) and the output
  // index to the last output
  constexpr int OPT = (G * D + NT - 1) / NT;               // outputs per thread
  constexpr int PF = OPT <= 2 ? 32 : 64 / OPT;             // partials prefetched per output
  float pre[OPT][PF];
#pragma unroll
  for (int u = 0; u < OPT; ++u) {
    const int idx = min(tid + NT * u, G * D - 1), h = idx / D, d = idx % D;
    const float* src = a.ws_acc + (pbase + (size_t)h * np) * D + d;
#pragma unroll
    for (int t8 = 0; t8 < PF; t8 += 8) {
      if (t8 < np) {
#pragma unroll
        for (int t = t8; t < t8 + 8; ++t) pre[u][t] = fetch(src + (size_t)min(t, np - 1) * D);
      } else {
#pragma unroll
        for (int t = t8; t < t8 + 8; ++t) pre[u][t] = 0.0f;
      }
    }
  }
  constexpr int HPW = (G + NW - 1) / NW;                   // heads per wave
  float mt[HPW], lt[HPW];
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int h = wave + NW * k;
    mt[k] = NEG_INF;
    lt[k] = 0.0f;
    if (h < G && lane < np) {
      const uint64_t ml = fetch_pair(a.ws_ml + 2 * (pbase + (size_t)h * np + lane));
      mt[k] = __builtin_bit_cast(float, (uint32_t)ml);
      lt[k] = __builtin_bit_cast(float, (uint32_t)(ml >> 32));
    }
  }
  // weights 2^(m_s - M) by DPP reductions over each half wave and a read of lanes 0
  // and 32 (by every lane: the half sums must be formed in both lanes)
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int h = wave + NW * k;
    if (h < G) {   // wave-uniform
      const float mh = lane_group_max<32>(mt[k]);
      const float M = fmaxf(readlane_f(mh, 0), readlane_f(mh, 32));
      const float w = mt[k] != NEG_INF ? fast_exp2(mt[k] - M) : 0.0f;
      const float lh = lane_group_sum<32>(w * lt[k]);
      const float L = readlane_f(lh, 0) + readlane_f(lh, 32);
      s_w[h * 64 + lane] = w;
      if (lane == 0) s_L[h] = L;
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < OPT; ++u) {
    const int idx = tid + NT * u;
    if (idx < G * D) {
      const int h = idx / D, d = idx % D;
      const float* wh = s_w + h * 64;
      float A = 0.0f;
#pragma unroll
      for (int t = 0; t < PF; ++t) A = __builtin_fmaf(pre[u][t], wh[t], A);
      for (int s0 = PF; s0 < np; s0 += PF) {   // the rest: PF loads issued together
        float x[PF];
#pragma unroll
        for (int t = 0; t < PF; ++t)
          x[t] = s0 + t < np ? fetch(a.ws_acc + (pbase + (size_t)h * np + s0 + t) * D + d) : 0.0f;
#pragma unroll
        for (int t = 0; t < PF; ++t)
          if (s0 + t < np) A = __builtin_fmaf(x[t], wh[s0 + t], A);
      }
      const float o = A / s_L[h];
      if (CODEC) s_out[h * D + d] = o;
      else a.out[(size_t)(b * a.Hq + kvh * G + h) * D + d] = o;
    }
  }
  if (CODEC) {   // back from the rotated domain: H o / sqrt(D), a row group per head
    __syncthreads();
    if (grp < G) {
      float v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) v[jj] = s_out[grp * D + 8 * c + jj];
      wht_row<LPR>(v, c);
      float* dst = a.out + (size_t)(b * a.Hq + kvh * G + grp) * D + 8 * c;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) dst[jj] = v[jj] * (1.0f / sqrtf((float)D));
    }
  }
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide max / sum for blockDim.x = D threads (1, 2 or 4 waves).
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* tmp) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float u = __shfl_xor(v, o);
    v = MAX ? fmaxf(v, u) : v + u;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) tmp[w] = v;
  __syncthreads();
  float r = tmp[0];
  const int nw = (blockDim.x + 63) >> 6;
  for (int i = 1; i < nw; ++i) r = MAX ? fmaxf(r, tmp[i]) : r + tmp[i];
  __syncthreads();
  return r;
}

// One workgroup of D threads per (query head, batch).  Thread d first requests dim d of
// the first PFM partials (one round trip; groups of 8 under a uniform test with the
// split index clamped, as in the in-kernel merge), then the (max, sum) pairs, staged in
// LDS; the weights 2^(m_s - M) follow from two block reductions, and thread d sums its
// prefetched partials (weights past ns are 0).  The codec's inverse rotation is one
// row transform by the first D/8 lanes.
template <int D, bool CODEC>
__global__ void __launch_bounds__(256) merge_kernel(DecodeArgs a) {
  constexpr int PFM = 64;
  __shared__ float s_w[MAX_SPLITS > PFM ? MAX_SPLITS : PFM];
  __shared__ float s_l[MAX_SPLITS];
  __shared__ float s_tmp[4];
  __shared__ float sh[D];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int ns = a.nsplit;
  const size_t base = (size_t)(b * a.Hq + h) * ns;
  const float* acc = a.ws_acc + base * D + d;
  float pre[PFM];
#pragma unroll
  for (int t8 = 0; t8 < PFM; t8 += 8) {
    if (t8 < ns) {
#pragma unroll
      for (int t = t8; t < t8 + 8; ++t) pre[t] = acc[(size_t)min(t, ns - 1) * D];
    } else {
#pragma unroll
      for (int t = t8; t < t8 + 8; ++t) pre[t] = 0.0f;
    }
  }
  float M = NEG_INF;
  for (int s = d; s < ns; s += D) {
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + 2 * (base + s));
    s_w[s] = ml.x;
    s_l[s] = ml.y;
    M = fmaxf(M, ml.x);
  }
  M = block_reduce<true>(M, s_tmp);
  float L = 0.0f;
  for (int s = d; s < max(ns, PFM); s += D) {
    float w = 0.0f;
    if (s < ns) {
      const float ms = s_w[s];
      w = ms != NEG_INF ? fast_exp2(ms - M) : 0.0f;
      L = __builtin_fmaf(w, s_l[s], L);
    }
    s_w[s] = w;
  }
  L = block_reduce<false>(L, s_tmp);   // its barrier also publishes s_w
  float A = 0.0f;
#pragma unroll
  for (int t = 0; t < PFM; ++t) A = __builtin_fmaf(pre[t], s_w[t], A);
  // more than PFM splits: 16 partials per step, their loads issued together
  constexpr int MU = 16;
  for (int s0 = PFM; s0 < ns; s0 += MU) {
    float x[MU];
#pragma unroll
    for (int u = 0; u < MU; ++u) x[u] = s0 + u < ns ? acc[(size_t)(s0 + u) * D] : 0.0f;
#pragma unroll
    for (int u = 0; u < MU; ++u)
      if (s0 + u < ns) A = __builtin_fmaf(x[u], s_w[s0 + u], A);
  }
  const float o = A / L;
  float* out = a.out + (size_t)(b * a.Hq + h) * D;
  if (CODEC) {   // back from the rotated domain: H o / sqrt(D), lane c holding dims 8c .. 8c + 7
    constexpr int LPR = D / 8;
    sh[d] = o;
    __syncthreads();
    if (d < LPR) {   // (LPR <= 32 consecutive lanes of the first wave, all active)
      float v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) v[jj] = sh[8 * d + jj];
      wht_row<LPR>(v, d);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) out[8 * d + jj] = v[jj] * (1.0f / sqrtf((float)D));
    }
  } else {
    out[d] = o;
  }
}

template <int D, int FMT>
hipError_t launch_d(const DecodeArgs& a, int G, hipStream_t s) {
  const dim3 grid(a.nsplit, a.Hkv, a.B);
  hipError_t e;
  if (FMT == KVQ_INT4_G && mfma_int4_eligible(D, a.gk, a.gv, a.cap, G))
    return launch_decode_int4_mfma(a, G, s);   // merges the splits itself
  if (FMT == KVQ_INT4_G16 && a.sinks == 0 && a.recent == 0 && mfma_int4_eligible(D, a.gk, a.gv, a.cap, G))
    return launch_decode_int4h_mfma(a, G, s);
  if (FMT == KVQ_INT8_TOKEN && mfma_int8_eligible(D, a.cap, G))
    return launch_decode_int8_mfma(a, G, s);
  // up to MERGE_INLINE_MAX splits the last split of a unit merges inside the kernel
  // (one launch less); more partials are merged by the merge kernel, which spreads
  // them over one workgroup per query head
  DecodeArgs k = a;
  k.merge_inline = a.nsplit <= MERGE_INLINE_MAX;
  switch (G) {
    case 1: e = launch_kernel(decode_splitk_kernel<D, 1, FMT>, grid, dim3(splitk_threads(D, FMT)), k, s); break;
    case 2: e = launch_kernel(decode_splitk_kernel<D, 2, FMT>, grid, dim3(splitk_threads(D, FMT)), k, s); break;
    case 4: e = launch_kernel(decode_splitk_kernel<D, 4, FMT>, grid, dim3(splitk_threads(D, FMT)), k, s); break;
    case 8: e = launch_kernel(decode_splitk_kernel<D, 8, FMT>, grid, dim3(splitk_threads(D, FMT)), k, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || k.merge_inline) return e;
  return launch_kernel(merge_kernel<D, FMT == KVQ_WHT_LM4 || FMT == KVQ_WHT_LM3>, dim3(a.Hq, a.B),
                       dim3(D), k, s);
}

template <int D>
hipError_t launch_fmt(int32_t format, const DecodeArgs& a, int G, hipStream_t s) {
  switch (format) {
    case KVQ_INT4_G: return launch_d<D, KVQ_INT4_G>(a, G, s);
    case KVQ_INT8_TOKEN: return launch_d<D, KVQ_INT8_TOKEN>(a, G, s);
    case KVQ_WHT_LM4: return launch_d<D, KVQ_WHT_LM4>(a, G, s);
    case KVQ_WHT_LM3: return launch_d<D, KVQ_WHT_LM3>(a, G, s);
    case KVQ_INT4_G16: return launch_d<D, KVQ_INT4_G16>(a, G, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int32_t plan_splits(const kvq_cache_desc* d, int32_t q_group, int32_t span) {
  const int32_t units = d->batch * d->kv_heads;
  if (units <= 0 || span <= 0) return 0;
  if (d->format == KVQ_INT4_G &&
      mfma_int4_eligible(d->head_dim, d->group_k, d->group_v, d->capacity, q_group))
    return plan_splits_mfma(units, span);
  if (d->format == KVQ_INT8_TOKEN && mfma_int8_eligible(d->head_dim, d->capacity, q_group))
    return plan_splits_mfma(units, span);
  if (mfma_int4h_eligible(d, q_group)) return plan_splits_mfma(units, span);
  // the codecs and INT4 with fp16 scales keep one more split for the new row when the
  // append is fused (planned for every call of those formats, so that the workspace
  // query does not depend on the call)
  const int32_t extra = is_codec(d->format) || d->format == KVQ_INT4_G16 ? 1 : 0;
  // workgroups: 4 per CU on 256 CUs (all resident), and positions per split worth a
  // workgroup (short contexts need many splits to fill the chip); the codecs at D = 256
  // run 512-thread workgroups (splitk_threads): half the workgroups, twice the rows
  const bool wide = is_codec(d->format) && d->head_dim == 256;
  const int32_t target = wide ? 512 : 1024;
  const int32_t min_rows = wide ? 128 : 64;
  int32_t n = (target + units - 1) / units - extra;
  const int32_t by_span = (span + min_rows - 1) / min_rows;
  if (n > by_span) n = by_span;
  if (n > 1024 - extra) n = 1024 - extra;
  return (n < 1 ? 1 : n) + extra;
}

hipError_t launch_decode(int32_t format, const DecodeArgs& a, int32_t q_group, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_fmt<64>(format, a, q_group, s);
    case 128: return launch_fmt<128>(format, a, q_group, s);
    case 256: return launch_fmt<256>(format, a, q_group, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
