// Top-k selection of one token's logits by one wave64, shared by the routing
// kernels (route.hip, and the fused routing + permutation kernels in
// permute.hip).
//
// Definition: the k experts with the largest fp32 logits, larger first, equal
// logits to the lower expert id, -0 equal to +0; slot j holds the j-th
// selection. Weights: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k
// selected logits, the sum taken in slot order: the full-softmax normaliser
// cancels in the renormalisation (page "TRTLLM-Gen MoE routing optimisation
// in FlashInfer: relieving register pressure", flashinfer PR #3751: the
// routing kernel's "softmax_sum" method, softmax then top-k then renormalise).
//
// A lane holds VPL of the token's logits in registers (VPL = E / 64 rounded
// up to a power of two: the compile-time tiers of that page's section 2).
// Entry i of a lane is expert lane + 64 i, or with VEC (16-byte loads, E a
// multiple of 4) expert 4 (lane + 64 (i / 4)) + i % 4. Entries past E hold
// -inf and are never selected (k <= E).
#pragma once

#include "device.h"

namespace moe {
namespace sel {

// Order-preserving unsigned image of a logit (-0 folded onto +0): larger
// logit, larger value. -inf maps to 0x007FFFFF, below every finite logit.
__device__ __forceinline__ uint32_t mono(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_mono(uint32_t m) {
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
}

template <bool VEC>
__device__ __forceinline__ uint32_t expert_of(int lane, int i) {
  return VEC ? 4 * (lane + kWave * (i / 4)) + (i % 4) : lane + kWave * i;
}

template <int VPL, bool VEC>
__device__ __forceinline__ void load_logits(const float* __restrict__ l, int lane, int E,
                                            float (&v)[VPL]) {
  if constexpr (VEC) {
    static_assert(VPL % 4 == 0, "groups of 4");
#pragma unroll
    for (int g = 0; g < VPL / 4; ++g) {
      const int e = 4 * (lane + kWave * g);
      const f32x4 q = e < E ? *reinterpret_cast<const f32x4*>(l + e)
                            : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * g + c] = q[c];
    }
  } else {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      v[i] = e < E ? l[e] : -INFINITY;
    }
  }
}

// Selection by k rounds of a wave-wide maximum. Every lane keeps the two best
// of its entries not yet taken (h1 before h2: larger value first, then lower
// expert). A round takes the wave maximum of the h1 values; when several
// lanes hold it, the lowest of their experts (a second reduction, skipped
// when one lane holds it). The winning lane moves h2 up, and when it wins a
// second time (its h2 already moved up) it rescans its entries after the one
// just taken. A lane's entries are visited in increasing expert order, so
// "greater than" keeps the lower expert on ties. Lane j ends with slot j
// (mine_v: image of the logit, mine_e: expert); top_v is slot 0's image.
template <int VPL, bool VEC>
__device__ __forceinline__ void select_rounds(const float (&v)[VPL], int lane, int E, int k,
                                              uint32_t& mine_v, uint32_t& mine_e,
                                              uint32_t& top_v) {
  uint32_t val[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) val[i] = (int)expert_of<VEC>(lane, i) < E ? mono(v[i]) : 0u;
  uint32_t h1v = 0, h1e = 0, h2v = 0, h2e = 0;
  auto top2 = [&](bool bounded, uint32_t bv, uint32_t be) {
    h1v = 0;
    h2v = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const uint32_t e = expert_of<VEC>(lane, i);
      uint32_t x = val[i];
      if (bounded) x = (x < bv || (x == bv && e > be)) ? x : 0u;
      const bool c1 = x > h1v, c2 = x > h2v;
      h2v = c1 ? h1v : (c2 ? x : h2v);
      h2e = c1 ? h1e : (c2 ? e : h2e);
      h1v = c1 ? x : h1v;
      h1e = c1 ? e : h1e;
    }
  };
  top2(false, 0u, 0u);
  bool h2_fresh = true;  // h2 is this lane's second best below h1
  mine_v = mine_e = top_v = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t m = wave_max_u32(h1v);
    const bool cand = h1v == m;
    const uint64_t cm = __builtin_amdgcn_ballot_w64(cand);
    uint32_t be;
    bool win;
    if (__builtin_popcountll(cm) == 1) {
      be = __builtin_amdgcn_readlane(static_cast<int>(h1e), __builtin_ctzll(cm));
      win = cand;
    } else {
      be = wave_min_u32(cand ? h1e : 0xFFFFFFFFu);
      win = cand && h1e == be;
    }
    if (j == 0) top_v = m;
    if (lane == j) {
      mine_v = m;
      mine_e = be;
    }
    const bool rescan = win && !h2_fresh;
    if (win) {
      h1v = h2v;
      h1e = h2e;
      h2_fresh = false;
    }
    if (__builtin_amdgcn_ballot_w64(rescan)) {
      if (rescan) {
        top2(true, m, be);
        h2_fresh = true;
      }
    }
  }
}

// Maximum over the 16 lanes of each row, in every lane of the row.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x121>(v));
  v = max(v, dpp_u32<0x122>(v));
  v = max(v, dpp_u32<0x124>(v));
  v = max(v, dpp_u32<0x128>(v));
  return v;
}

// Selection by a threshold. In each 16-lane row, r = the q-th largest of the
// row's lane maxima (counted with multiplicity), q = ceil(k / 4): the row holds
// q distinct entries >= r. The four rows hold disjoint entries, so at least
// 4 q >= k entries are >= tau = the smallest of the four r, and tau is at most
// the k-th largest logit. Every entry >= tau is a candidate (k of them at
// least, usually a few more); the candidates are compacted into the wave's LDS
// row `cand` (64 keys) as (image << 32 | ~expert), so a larger key is an
// earlier slot, and each candidate's slot is the number of larger keys.
// Returns false, with nothing selected, when more than 64 entries lie at or
// above tau (ties; select_rounds handles that case). Outputs as
// select_rounds.
template <int VPL, bool VEC>
__device__ __forceinline__ bool select_threshold(const float (&v)[VPL], int lane, int k,
                                                 unsigned long long* cand, uint32_t& mine_v,
                                                 uint32_t& mine_e, uint32_t& top_v) {
  float m = v[0];
#pragma unroll
  for (int i = 1; i < VPL; ++i) m = fmaxf(m, v[i]);
  uint32_t x = mono(m);
  const int q = (k + 3) / 4;
  const int rshift = 16 * (lane / 16);
  int need = q;
  uint32_t r = 0;  // the row's threshold, 0 until found
  for (int it = 0; it < q; ++it) {  // a row that has not found r has >= need lanes left
    const uint32_t mx = row_max_u32(x);
    const uint64_t bm = __builtin_amdgcn_ballot_w64(x == mx);
    const int c = __builtin_popcount(static_cast<uint32_t>(bm >> rshift) & 0xFFFFu);
    if (r == 0) {
      if (c >= need) r = mx;
      need -= c;
      x = x == mx ? 0u : x;
    }
  }
  const uint32_t tau =
      min(min(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(r), 0)),
              static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(r), 16))),
          min(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(r), 32)),
              static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(r), 48))));
  if (tau < 0x00800000u) return false;  // a row without q finite maxima (select_rounds)
  const float tf = from_mono(tau);
  int n = 0;  // candidates so far (wave-uniform)
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const bool c = v[i] >= tf;
    const uint64_t bm = __builtin_amdgcn_ballot_w64(c);
    if (bm) {
      const int pos = n + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bm >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bm), 0));
      if (c && pos < kWave)
        cand[pos] = (static_cast<unsigned long long>(mono(v[i])) << 32) |
                    (0xFFFFFFFFu - expert_of<VEC>(lane, i));
      n += __builtin_popcountll(bm);
    }
  }
  if (n > kWave) return false;
  __builtin_amdgcn_wave_barrier();
  const unsigned long long key = lane < n ? cand[lane] : 0ull;
  int rank = 0;
  for (int j = 0; j < n; ++j) rank += cand[j] > key ? 1 : 0;
  __builtin_amdgcn_wave_barrier();
  // every lane has read the candidates (in-order LDS within the wave); slot r
  // of the row now receives the key ranked r
  if (lane < n && rank < k) cand[rank] = key;
  __builtin_amdgcn_wave_barrier();
  const unsigned long long mine = lane < k ? cand[lane] : 0ull;
  mine_v = static_cast<uint32_t>(mine >> 32);
  mine_e = 0xFFFFFFFFu - static_cast<uint32_t>(mine);
  top_v = static_cast<uint32_t>(cand[0] >> 32);
  __builtin_amdgcn_wave_barrier();
  return true;
}

// Selection and weights of one token whose logits the wave holds in v; lanes
// j < k write slot j of ids / weights (row t) and return its expert.
// THRESH: try select_threshold first (tiers of 4 and more values per lane).
template <int VPL, bool VEC, bool THRESH>
__device__ __forceinline__ uint32_t route_token(const float (&v)[VPL], int lane, int E, int k,
                                                unsigned long long* cand, int* __restrict__ ids,
                                                float* __restrict__ weights, size_t t) {
  uint32_t mine_v = 0, mine_e = 0, top_v = 0;
  bool done = false;
  if constexpr (THRESH) done = select_threshold<VPL, VEC>(v, lane, k, cand, mine_v, mine_e, top_v);
  if (!done) select_rounds<VPL, VEC>(v, lane, E, k, mine_v, mine_e, top_v);
  const float topf = from_mono(top_v);
  const float ex = lane < k ? expf(from_mono(mine_v) - topf) : 0.0f;
  float s = 0.0f;  // sum in slot order
  for (int j = 0; j < k; ++j)
    s += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), j));
  if (lane < k) {
    ids[t * k + lane] = static_cast<int>(mine_e);
    weights[t * k + lane] = ex / s;
  }
  return mine_e;
}

}  // namespace sel
}  // namespace moe
