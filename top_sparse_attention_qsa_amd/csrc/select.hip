// select.hip -- steps 2-5: top-k membership, chronological emission, group
// expansion and tail append for every row.
//
// Membership follows the total order (score descending, group position
// ascending); ties are settled while the set is chosen, never after it is
// sorted (AFN-017 "Top-k chooses the set; time chooses the order", §Decision
// and §Tie handling belongs to membership).  The chosen groups leave in
// ascending logical position, each as four consecutive token IDs, followed
// by the raw tail (same note, §Decision; §The dense-parity property).
//
// One 1024-thread workgroup per row:
//  1. tau = the k-th largest of the per-16-group maxima (when there are at
//     least k of them).  Those k maxima are k distinct groups scoring >= tau,
//     so the k-th largest score is >= tau and every member scores >= tau.
//  2. One streaming pass compacts the candidates (score >= tau) in position
//     order into LDS.  If more than kCandCap survive (massive ties), the
//     passes below stream the whole row from global memory instead.
//  3. A byte-wise radix select over the order keys finds T, the k-th largest
//     key, and the number of keys above T.  Candidates lie between tau and
//     the row's largest key, so it starts below the bits those two share.
//  4. An ordered pass keeps every key above T and the first (k - above)
//     keys equal to T in position order -- the tie rule -- and writes each
//     kept group at its output index, which is already chronological.
// Causal-chunk rows (select_certified_kernel) hold upper bounds of the chain
// scores instead; between steps 2 and 3 their candidates are settled by
// bounds where possible and the rest rescored exactly (CertifiedScores).
// No sort, no float atomics; the result is unique, so it is bit-identical to
// any correct selector.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int NT = kSelectThreads;
constexpr int NWAVES = NT / kWave;

constexpr int kMaxStage = 4096;   // segment maxima staged in LDS (G <= 65,536)
constexpr int kPerThread = 32;    // scores held per thread in one streaming pass

struct alignas(16) SelectShared {
  uint32_t hist[3][256];  // radix passes rotate through three histograms
  uint32_t wave_tot[NWAVES];
  uint32_t wave_aux[NWAVES];  // a second per-wavefront value (certified rows)
  uint32_t counter;
  uint32_t cand_key[kCandCap];
  uint32_t cand_pos[kCandCap];
  uint32_t maxima[kMaxStage];
};

// Histogram add in which lanes of a wavefront that share a bin are first
// merged (up to two bins peeled per call), so a skewed digit does not
// serialise 64 LDS atomics on one address.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
  const int lane = lane_id();
  uint64_t pending = __ballot(active);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    if (pending == 0) return;
    const int leader = __ffsll((unsigned long long)pending) - 1;
    const uint32_t lb = lane_value(bin, leader);
    const uint64_t same = __ballot(active && bin == lb);
    if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
    if ((same >> lane) & 1ull) active = false;
    pending &= ~same;
  }
  if (active) atomicAdd(&hist[bin], 1u);
}

// k-th largest order key among the n keys from src whose top `known` bits
// equal those of `prefix0` (every key when known = 0; the caller guarantees
// that every other key is smaller), and the count of those keys strictly
// above it.  The next `resolve` bits are settled in 8-bit digits, most
// significant first; a last digit that reaches below bit 0 is taken at bits
// 0..7 instead, overlapping bits already settled, which every remaining key
// matches.  Bits below the settled ones come back cleared: the result is then
// a lower bound of the k-th largest key, and the count is that of keys above
// the settled prefix.  Returns false -- after a barrier, leaving the outputs
// unwritten -- when fewer than k keys share the known prefix.
//
// One barrier per pass: every wavefront finds the digit from the pass's
// histogram itself (the same values, so the same digit), and the passes
// rotate through three histograms, so the one a pass clears for its
// successor was last read two passes earlier, before the previous pass's
// barrier.  On entry no wavefront may still read sh.hist (the caller has
// passed a barrier since the last call).
template <class Src>
__device__ bool radix_kth_largest(const Src& src, uint32_t n, uint32_t k, SelectShared& sh,
                                  uint32_t* t_out, uint32_t* above_out, uint32_t prefix0 = 0,
                                  int known = 0, int resolve = 32) {
  const int tid = (int)threadIdx.x;
  const int lane = lane_id();
  uint32_t mask = known > 0 ? ~0u << (32 - known) : 0u;
  uint32_t prefix = prefix0 & mask, kk = k, above = 0;
  const int passes = (resolve + 7) / 8;
  for (int i = tid; i < 256; i += NT) sh.hist[0][i] = 0;
  __syncthreads();
#pragma unroll 1
  for (int p = 0; p < passes; ++p) {
    const int top = 32 - known - 8 * p;          // bits >= top are settled
    const int shift = top > 8 ? top - 8 : 0;
    uint32_t* hist = sh.hist[p % 3];
    if (p + 1 < passes)
      for (int i = tid; i < 256; i += NT) sh.hist[(p + 1) % 3][i] = 0;
    const uint32_t n_up = (n + NT - 1) / NT * NT;   // whole wavefronts stay converged
    for (uint32_t i = tid; i < n_up; i += NT) {
      bool act = false;
      uint32_t bin = 0;
      if (i < n) {
        const uint32_t key = src.key(i);
        act = (key & mask) == prefix;
        bin = (key >> shift) & 255u;
      }
      hist_add(hist, bin, act);
    }
    __syncthreads();
    // lane l owns bins 4l..4l+3; the lane whose bins hold the kk-th largest
    // finds the digit, which every lane then reads from it
    const uint4 h = *reinterpret_cast<const uint4*>(hist + 4 * lane);
    const uint32_t mine = (h.x + h.y) + (h.z + h.w);
    const uint32_t inc = wave_inclusive_sum(mine);  // lanes <= l
    const uint32_t total = lane_value(inc, kWave - 1);
    if (p == 0 && total < kk) {
      __syncthreads();  // every wavefront is done reading this histogram
      return false;
    }
    const uint32_t higher = total - inc;    // keys in bins above lane l's
    const uint32_t suffix = higher + mine;  // keys in lane l's bins and above
    const bool owner = higher < kk && kk <= suffix;
    uint32_t acc = higher, digit = 4u * (uint32_t)lane;
    const uint32_t hb[4] = {h.x, h.y, h.z, h.w};
    bool found = false;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      if (!found && acc + hb[b] >= kk) {
        digit = 4u * (uint32_t)lane + (uint32_t)b;
        found = true;
      }
      if (!found) acc += hb[b];
    }
    const int src_lane = __ffsll((unsigned long long)__ballot(owner)) - 1;
    digit = lane_value(digit, src_lane);
    acc = lane_value(acc, src_lane);
    above += acc;
    kk -= acc;
    prefix |= digit << shift;
    mask |= 255u << shift;
  }
  *t_out = prefix;
  *above_out = above;
  return true;
}

struct GlobalScores {
  const float* s;
  __device__ uint32_t key(uint32_t i) const { return order_key(s[i]); }
};
struct GlobalKeys {
  const uint32_t* k;
  __device__ uint32_t key(uint32_t i) const { return k[i]; }
};
struct LdsCands {
  const uint32_t* k;
  __device__ uint32_t key(uint32_t i) const { return k[i]; }
};

// Policy of the plain (decode) selection: the row's scores are exact.
struct PlainScores {
  static constexpr bool kCertified = false;
  const float* srow;
  __device__ uint32_t full_key(uint32_t g) const { return order_key(srow[g]); }
  __device__ uint32_t exact_key(uint32_t g) const { return order_key(srow[g]); }
};

// Policy of the certified (chunk) selection: the row's "scores" are upper
// bounds hi = s~ + E of the chain scores (chunk.hip), so candidates are
// rescored here with the chain itself -- the same fused multiply-adds, in the
// same order, as score.hip -- before the exact selection.
template <int HI, int DI>
struct CertifiedScores {
  static constexpr bool kCertified = true;
  const float* q;    // this row's index query [HI][DI]
  const float* kp;   // this sequence's tiled pooled keys
  const float* wrow; // this row's tile widths (chunk.hip), may be null
  __device__ uint32_t exact_key(uint32_t g) const {
    const float* kb = kp + (int64_t)(g >> 6) * (64 * DI) + (g & 63) * 4;
    float acc[HI];
#pragma unroll
    for (int h = 0; h < HI; ++h) acc[h] = 0.0f;
#pragma unroll 4
    for (int c = 0; c < DI / 4; ++c) {
      const float4 kv = *reinterpret_cast<const float4*>(kb + c * 256);
#pragma unroll
      for (int h = 0; h < HI; ++h) {
        float a = acc[h];
        a = __builtin_fmaf(q[h * DI + 4 * c + 0], kv.x, a);
        a = __builtin_fmaf(q[h * DI + 4 * c + 1], kv.y, a);
        a = __builtin_fmaf(q[h * DI + 4 * c + 2], kv.z, a);
        a = __builtin_fmaf(q[h * DI + 4 * c + 3], kv.w, a);
        acc[h] = a;
      }
    }
    float sc = 0.0f;
#pragma unroll
    for (int h = 0; h < HI; ++h) sc = sc + (acc[h] > 0.0f ? acc[h] : 0.0f);
    return order_key(sc);
  }
  __device__ uint32_t full_key(uint32_t g) const { return exact_key(g); }

  // Exact keys of the n compacted candidates, written over their bounds: a
  // wavefront takes 64 candidates at a time, lane = candidate, and runs the
  // chain on v_mfma_f32_4x4x1_16b_f32 exactly as score.hip does (one
  // rounding per step, so the bits are those of exact_key).  The query row is
  // staged in `qs` (LDS scratch of DI * HI floats, dimension-major: entry
  // (d, i) holds heads i, 4+i, ...).  Called by the whole workgroup.
  __device__ void rescore_all(uint32_t* cand_key, const uint32_t* cand_pos, uint32_t n,
                              float* qs, const uint32_t* idx = nullptr) const {
    static_assert(HI % 4 == 0, "head quads");
    constexpr int HQ = HI / 4;
    constexpr int NC = DI / 4;
    // a candidate's key is 32 pieces of 16 B, 1 KiB apart in the tiled layout:
    // up to 16 gathers in flight per lane (4 in flight: 210 us of rescoring
    // per causal-chunk leg, 16: 188 us, against 253 us for one chain per
    // thread on the VALU)
    constexpr int PF = 16 < NC ? 16 : NC;
    typedef float v4f __attribute__((ext_vector_type(4)));
    typedef float vqf __attribute__((ext_vector_type(HQ)));
    const int tid = (int)threadIdx.x;
    for (int e = tid; e < DI * 4; e += NT) {
      const int d = e >> 2, i = e & 3;
      vqf v;
#pragma unroll
      for (int m = 0; m < HQ; ++m) v[m] = q[(4 * m + i) * DI + d];
      *reinterpret_cast<vqf*>(qs + e * HQ) = v;
    }
    __syncthreads();
    const int lane = lane_id();
    const int qi = lane & 3;
    for (uint32_t base = 64u * (uint32_t)wave_id(); base < n; base += 64u * NWAVES) {
      const uint32_t j = base + (uint32_t)lane;
      const bool valid = j < n;
      // candidate j of the list (idx) or of the whole compaction; n >= 1, so
      // lanes past n reread entry 0
      const uint32_t c_i = idx ? idx[valid ? j : 0u] : (valid ? j : 0u);
      const uint32_t g = cand_pos[c_i];
      const float* kb = kp + (int64_t)(g >> 6) * (64 * DI) + (g & 63) * 4;
      float4 ring[PF];
#pragma unroll
      for (int u = 0; u < PF; ++u) ring[u] = *reinterpret_cast<const float4*>(kb + u * 256);
      v4f acc[HQ];
#pragma unroll
      for (int m = 0; m < HQ; ++m) acc[m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float4 kv = ring[c % PF];
        if (c + PF < NC) ring[c % PF] = *reinterpret_cast<const float4*>(kb + (c + PF) * 256);
        const vqf a0 = *reinterpret_cast<const vqf*>(qs + ((4 * c + 0) * 4 + qi) * HQ);
        const vqf a1 = *reinterpret_cast<const vqf*>(qs + ((4 * c + 1) * 4 + qi) * HQ);
        const vqf a2 = *reinterpret_cast<const vqf*>(qs + ((4 * c + 2) * 4 + qi) * HQ);
        const vqf a3 = *reinterpret_cast<const vqf*>(qs + ((4 * c + 3) * 4 + qi) * HQ);
#pragma unroll
        for (int m = 0; m < HQ; ++m) acc[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(a0[m], kv.x, acc[m], 0, 0, 0);
#pragma unroll
        for (int m = 0; m < HQ; ++m) acc[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(a1[m], kv.y, acc[m], 0, 0, 0);
#pragma unroll
        for (int m = 0; m < HQ; ++m) acc[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(a2[m], kv.z, acc[m], 0, 0, 0);
#pragma unroll
        for (int m = 0; m < HQ; ++m) acc[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(a3[m], kv.w, acc[m], 0, 0, 0);
      }
      float sc = 0.0f;
#pragma unroll
      for (int m = 0; m < HQ; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc = sc + (acc[m][i] > 0.0f ? acc[m][i] : 0.0f);
      if (valid) cand_key[c_i] = order_key(sc);
    }
  }
};

template <class P>
struct FullKeys {
  const P* pol;
  __device__ uint32_t key(uint32_t i) const { return pol->full_key(i); }
};

// The float an order key came from (-0 comes back as +0).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Writes kept group g at output index o: token IDs 4g..4g+3 at 4o, and/or
// bit g of the bitmap.
struct Emitter {
  int32_t* ids;        // row of 4k+4, may be null
  uint32_t* bitmap;    // row of g_max/32 words, may be null
  uint32_t k;
  __device__ void keep(uint32_t o, uint32_t g) const {
    if (ids && o < k) {
      const int32_t t = (int32_t)(4u * g);
      *reinterpret_cast<int4*>(ids + 4 * o) = make_int4(t, t + 1, t + 2, t + 3);
    }
    if (bitmap) atomicOr(&bitmap[g >> 5], 1u << (g & 31));
  }
};

// Candidate compaction that reads only the segments that can hold a member
// (decode rows, whose scores are exact).  Each thread owns the maxima of four
// consecutive segments in registers; tau = a lower bound of the k-th largest
// of the (folded) maxima, from a two-pass radix select on their top 16 bits.
// A segment whose maximum is below tau holds no group scoring >= tau, so each
// wavefront lists, in order, the segments of its span (256 segments) that
// reach tau and reads only their scores, 64 at a time (four segments per
// load instruction).  Scores >= tau are compacted in position order into LDS:
// wavefront order, then round order, then lane order, which is position
// order.  Returns false, having changed nothing but LDS, when a wavefront
// lists more than kSegRounds*4 segments; sets *overflow when more than
// kCandCap candidates survive.
constexpr int kSegRounds = 16;  // 64-score rounds per wavefront in one pass

__device__ bool segment_candidates(SelectShared& sh, const float* __restrict__ srow,
                                   const uint32_t* __restrict__ mrow, uint32_t G, uint32_t segs,
                                   uint32_t k, uint32_t* n_cand, bool* overflow,
                                   uint32_t* tau_out, uint32_t* top_out) {
  const int tid = (int)threadIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();
  const uint32_t s0 = 4u * (uint32_t)tid;
  uint32_t mx[4];
  if (s0 + 4 <= segs) {
    const uint4 v = *reinterpret_cast<const uint4*>(mrow + s0);
    mx[0] = v.x; mx[1] = v.y; mx[2] = v.z; mx[3] = v.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) mx[e] = (s0 + e < segs) ? mrow[s0 + e] : 0u;
  }
  // fold f neighbouring maxima into one while at least 2k values remain; each
  // folded value is still the maximum of a disjoint set of groups
  uint32_t f = 1;
  while (f < 4 && (segs / (2 * f)) >= 2u * k) f *= 2;
  const uint32_t nf = (segs + f - 1) / f;
  if (f == 4) {
    const uint32_t a = mx[0] > mx[1] ? mx[0] : mx[1], b = mx[2] > mx[3] ? mx[2] : mx[3];
    if (s0 / 4 < nf) sh.maxima[s0 / 4] = a > b ? a : b;
  } else if (f == 2) {
    if (s0 / 2 < nf) sh.maxima[s0 / 2] = mx[0] > mx[1] ? mx[0] : mx[1];
    if (s0 / 2 + 1 < nf) sh.maxima[s0 / 2 + 1] = mx[2] > mx[3] ? mx[2] : mx[3];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (s0 + e < nf) sh.maxima[s0 + e] = mx[e];
  }
  // the row's largest key, the largest segment maximum (sh.wave_tot is free
  // until the listing below)
  {
    const uint32_t a = mx[0] > mx[1] ? mx[0] : mx[1], b = mx[2] > mx[3] ? mx[2] : mx[3];
    const uint32_t r = row_max16_u32(a > b ? a : b);
    // readlane returns int: compare the lanes' keys as unsigned
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)r, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)r, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)r, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)r, 48);
    const uint32_t r01 = r0 > r1 ? r0 : r1, r23 = r2 > r3 ? r2 : r3;
    if (lane == 0) sh.wave_tot[wave] = r01 > r23 ? r01 : r23;
  }
  __syncthreads();
  uint32_t top = 0;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) top = top > sh.wave_tot[w] ? top : sh.wave_tot[w];
  // tau: the k-th largest maximum to 17 bits in one pass, among the maxima
  // sharing the largest one's sign and exponent (9 bits) -- all maxima
  // outside that binade are smaller; or, when fewer than k share it, to 16
  // bits in two passes over all of them.  Either way a lower bound of the
  // k-th largest maximum.
  uint32_t tau, above_unused;
  if (!radix_kth_largest(LdsCands{sh.maxima}, nf, k, sh, &tau, &above_unused, top, 9, 8))
    radix_kth_largest(LdsCands{sh.maxima}, nf, k, sh, &tau, &above_unused, 0u, 0, 16);
  *tau_out = tau;
  *top_out = top;

  // this wavefront's list of segments reaching tau (in sh.maxima, 256 per
  // wavefront, after the radix select is done with it)
  uint32_t fl = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (s0 + e < segs && mx[e] >= tau) fl |= 1u << e;
  const uint32_t c = (uint32_t)__popc(fl);
  const uint64_t b0 = __ballot(c & 1u), b1 = __ballot(c & 2u), b2 = __ballot(c & 4u);
  uint32_t o = lanes_below(b0) + 2u * lanes_below(b1) + 4u * lanes_below(b2);
  const uint32_t nseg = (uint32_t)(__popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2));
  uint32_t* wlist = sh.maxima + 256 * wave;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if ((fl >> e) & 1u) wlist[o++] = s0 + e;
  // (the list is written and read by this wavefront only)

  // rounds of 64 scores: item i = 64r + lane is score i%16 of listed segment
  // i/16.  Every round's load is issued before any result is used (a load
  // behind a branch, or used at once, would be waited for before the next
  // one is issued: one memory round trip per round); items past the list
  // read position 0 and are masked afterwards.
  const uint32_t items = nseg * kSegment;
  uint32_t key[kSegRounds], pos[kSegRounds];
  uint64_t hit[kSegRounds];
  uint32_t cnt = 0;
  {
    float sval[kSegRounds];
    bool valid[kSegRounds];
#pragma unroll
    for (int r = 0; r < kSegRounds; ++r) {
      const uint32_t i = 64u * r + (uint32_t)lane;
      const bool in = i < items;
      const uint32_t sg = wlist[in ? i / kSegment : 0];
      pos[r] = sg * kSegment + (i % kSegment);
      valid[r] = in && pos[r] < G;
      sval[r] = srow[valid[r] ? pos[r] : 0u];
    }
#pragma unroll
    for (int r = 0; r < kSegRounds; ++r) key[r] = valid[r] ? order_key(sval[r]) : 0u;
  }
#pragma unroll
  for (int r = 0; r < kSegRounds; ++r) {
    const uint32_t i = 64u * r + (uint32_t)lane;
    hit[r] = __ballot(i < items && pos[r] < G && key[r] >= tau);
    cnt += (uint32_t)__popcll(hit[r]);
  }
  const bool too_many = items > 64u * kSegRounds;
  if (lane == 0) sh.wave_tot[wave] = too_many ? 0xFFFFFFFFu : cnt;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  bool any_too_many = false;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    const uint32_t t = sh.wave_tot[w];
    any_too_many |= t == 0xFFFFFFFFu;
    base += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();  // wave_tot is reused by later scans
  if (any_too_many) return false;
  if (tot > (uint32_t)kCandCap) {
    *overflow = true;
    return true;
  }
#pragma unroll
  for (int r = 0; r < kSegRounds; ++r) {
    if ((hit[r] >> lane) & 1ull) {
      const uint32_t at = base + lanes_below(hit[r]);
      sh.cand_key[at] = key[r];
      sh.cand_pos[at] = pos[r];
    }
    base += (uint32_t)__popcll(hit[r]);
  }
  *n_cand = tot;
  return true;
}

template <class P>
__device__ void select_row(const P& pol, SelectShared& sh, const float* __restrict__ scores,
                           const uint32_t* __restrict__ maxima, const RowView& rv, int64_t lrow,
                           int64_t row, int64_t g_max, int32_t k, uint32_t* __restrict__ bitmap,
                           int32_t* __restrict__ token_ids, int32_t* __restrict__ width) {
  const int tid = (int)threadIdx.x;
  const int32_t stride = 4 * k + 4;
  int32_t* ids = token_ids ? token_ids + row * stride : nullptr;
  uint32_t* bm = bitmap ? bitmap + row * (g_max / 32) : nullptr;

  if (bm) {
    const int64_t words = g_max / 32;
    for (int64_t w = tid; w < words; w += NT) bm[w] = 0u;
    __threadfence();
    __syncthreads();
  }
  if (!rv.valid) {
    if (ids)
      for (int i = tid; i < stride; i += NT) ids[i] = -1;
    if (width && tid == 0) width[row] = -1;
    return;
  }

  const uint32_t G = (uint32_t)rv.g;
  const Emitter em{ids, bm, (uint32_t)k};
  uint32_t kept;
  if (G <= (uint32_t)k) {
    // every complete group survives: the dense causal row
    for (uint32_t g = tid; g < G; g += NT) em.keep(g, g);
    kept = G;
  } else {
    const float* __restrict__ srow = scores + lrow * g_max;
    uint32_t n_cand = 0;
    bool overflow = false;
    bool compacted = false;  // candidates already in LDS (segment-skipping pass)
    // certified rows: this thread's share of the row's widest segment,
    // loaded here so the loads overlap the threshold and compaction
    float wpart = 0.0f;
    if constexpr (P::kCertified) {
      if (pol.wrow) {
        const uint32_t tiles_w = (G + 63) / 64;
        for (uint32_t t = tid; t < tiles_w; t += NT) wpart = fmaxf(wpart, pol.wrow[t]);
      }
    }
    uint32_t tau = 0, top = 0;  // with compacted: every candidate key is in [tau, top]
    const uint32_t segs = (G + kSegment - 1) / kSegment;
    if constexpr (!P::kCertified) {
      if (maxima && segs >= (uint32_t)k && segs <= 4u * NT)
        compacted = segment_candidates(sh, srow, maxima + lrow * (g_max / kSegment), G, segs,
                                       (uint32_t)k, &n_cand, &overflow, &tau, &top);
    }
    if (!compacted) {
    // 1. threshold bound from the segment maxima, staged once in LDS.  While
    //    at least 2k would remain, f neighbouring maxima are folded into one
    //    (their maximum): still one maximum per disjoint set of groups, so the
    //    k-th largest of the folded values is still a lower bound of the k-th
    //    largest score, and the radix select works on fewer values.
    tau = 0;
    if (maxima && segs >= (uint32_t)k) {
      const uint32_t* mrow = maxima + lrow * (g_max / kSegment);
      uint32_t f = 1;
      while (f < 8 && (segs / (2 * f)) >= 2u * (uint32_t)k) f *= 2;
      const uint32_t nf = (segs + f - 1) / f;
      uint32_t above_unused;
      if (nf <= (uint32_t)kMaxStage) {
        for (uint32_t i = tid; i < nf; i += NT) {
          uint32_t m = 0;
          for (uint32_t e = 0; e < f; ++e) {
            const uint32_t j = i * f + e;
            const uint32_t v = j < segs ? mrow[j] : 0u;
            m = m > v ? m : v;
          }
          sh.maxima[i] = m;
        }
        __syncthreads();
        radix_kth_largest(LdsCands{sh.maxima}, nf, (uint32_t)k, sh, &tau, &above_unused);
      } else {
        radix_kth_largest(GlobalKeys{mrow}, segs, (uint32_t)k, sh, &tau, &above_unused);
      }
    }
    // 2. ordered candidate compaction.  A pass covers kPerThread*NT positions;
    //    wavefront w owns a contiguous span of kPerThread*64 of them, read as
    //    kPerThread/4 coalesced 1 KiB float4 loads (lane l holds positions
    //    span + 256j + 4l .. +3).  Position order is (w, j, l, e), so a lane's
    //    output index is the workgroup prefix of the wavefront totals, plus the
    //    wavefront's running count over j, plus a bit-sliced ballot prefix over
    //    the lanes below it.
    constexpr int NJ = kPerThread / 4;
    const int lane = lane_id();
    const int wave = wave_id();
    for (uint32_t base = 0; base < G; base += (uint32_t)kPerThread * NT) {
      const uint32_t span = base + (uint32_t)wave * (kPerThread * kWave);
      uint32_t keys[kPerThread];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t p = span + 256u * j + 4u * lane;
        if (p + 4 <= G) {
          const float4 f4 = *reinterpret_cast<const float4*>(srow + p);
          keys[4 * j + 0] = order_key(f4.x);
          keys[4 * j + 1] = order_key(f4.y);
          keys[4 * j + 2] = order_key(f4.z);
          keys[4 * j + 3] = order_key(f4.w);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) keys[4 * j + e] = (p + e < G) ? order_key(srow[p + e]) : 0u;
        }
      }
      uint32_t flags = 0;  // bit 4j+e: position span + 256j + 4*lane + e is a candidate
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t p = span + 256u * j + 4u * lane + e;
          if (p < G && keys[4 * j + e] >= tau) flags |= 1u << (4 * j + e);
        }
      // per j: this lane's count c (0..4) and the count over lanes below it
      uint32_t below[NJ], wave_total = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t c = (uint32_t)__popc((flags >> (4 * j)) & 15u);
        const uint64_t b0 = __ballot(c & 1u), b1 = __ballot(c & 2u), b2 = __ballot(c & 4u);
        below[j] = wave_total + lanes_below(b0) + 2u * lanes_below(b1) + 4u * lanes_below(b2);
        wave_total += (uint32_t)(__popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2));
      }
      if (lane == 0) sh.wave_tot[wave] = wave_total;
      __syncthreads();
      uint32_t wave_base = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < NWAVES; ++w) {
        const uint32_t t = sh.wave_tot[w];
        wave_base += (w < wave) ? t : 0u;
        tot += t;
      }
      __syncthreads();
      if (n_cand + tot > (uint32_t)kCandCap) { overflow = true; break; }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        uint32_t o = n_cand + wave_base + below[j];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((flags >> (4 * j + e)) & 1u) {
            sh.cand_key[o] = keys[4 * j + e];
            sh.cand_pos[o] = span + 256u * j + 4u * lane + e;
            ++o;
          }
      }
      n_cand += tot;
    }
    }  // !compacted
    __syncthreads();
    if constexpr (P::kCertified) {
      // The candidates' keys are their upper bounds hi >= s (s: the chain
      // score).  With W >= hi - s for every group of the row (the widest
      // tile), fl(hi - W) <= s as well.  Let H_k and H_k1 be the k-th and
      // (k+1)-th largest hi.  A candidate with hi < fl(H_k - W) is beaten by
      // the k groups whose hi reaches H_k (their s >= fl(H_k - W)): it is
      // out.  One with fl(hi - W) > H_k1 can be beaten only by groups whose
      // hi exceeds H_k1, at most k of them counting itself: it is in.  Only
      // the rest -- a band around the k-th score -- is rescored exactly, with
      // the chain; "in" keys become the largest key, "out" keys 0 (below
      // every score's key), and the exact selection below then picks the same
      // set as the chain scores.  The query row is staged over the segment
      // maxima, which are no longer read, and the band list after it.
      if (!overflow) {
        static_assert(sizeof(SelectShared::maxima) >= sizeof(float) * 16 * 128 * 2,
                      "query staging and band list");
        float* qs = reinterpret_cast<float*>(sh.maxima);
        uint32_t* band = sh.maxima + 16 * 128;
        constexpr uint32_t kBandCap = kMaxStage - 16 * 128;
        bool all = pol.wrow == nullptr || n_cand <= (uint32_t)k;
        if (!all) {
          const int lane = lane_id(), wave = wave_id();
          // W: the row's widest tile
          const float ww = wave_max(wpart);
          if (lane == 0) sh.wave_aux[wave] = __float_as_uint(ww);
          if (tid == 0) sh.counter = 0u;
          uint32_t T1, above1;
          radix_kth_largest(LdsCands{sh.cand_key}, n_cand, (uint32_t)k, sh, &T1, &above1);
          float W = 0.0f;
#pragma unroll
          for (int w = 0; w < NWAVES; ++w) W = fmaxf(W, __uint_as_float(sh.wave_aux[w]));
          // keys equal to H_k, and the largest key below it
          uint32_t eq = 0u, below = 0u;
          for (uint32_t i = tid; i < n_cand; i += NT) {
            const uint32_t key = sh.cand_key[i];
            eq += key == T1 ? 1u : 0u;
            below = (key < T1 && key > below) ? key : below;
          }
          const uint32_t eq_w = (uint32_t)wave_sum_u32(eq);
          const uint32_t below_w = wave_max_u32(below);
          __syncthreads();  // every wavefront has read wave_aux (W)
          if (lane == 0) {
            sh.wave_tot[wave] = eq_w;
            sh.wave_aux[wave] = below_w;
          }
          __syncthreads();
          uint32_t eq_all = 0u, below_all = 0u;
#pragma unroll
          for (int w = 0; w < NWAVES; ++w) {
            eq_all += sh.wave_tot[w];
            below_all = sh.wave_aux[w] > below_all ? sh.wave_aux[w] : below_all;
          }
          const float hk = key_value(T1);
          const uint32_t T2 = above1 + eq_all > (uint32_t)k ? T1 : below_all;
          const float hk1 = T2 == 0u ? -INFINITY : key_value(T2);
          const float out_below = hk - W;
          for (uint32_t i = tid; i < n_cand; i += NT) {
            const float h = key_value(sh.cand_key[i]);
            if (h < out_below) {
              sh.cand_key[i] = 0u;
            } else if (h - W > hk1) {
              sh.cand_key[i] = 0xFFFFFFFFu;
            } else {
              const uint32_t slot = atomicAdd(&sh.counter, 1u);
              if (slot < kBandCap) band[slot] = i;
            }
          }
          __syncthreads();
          const uint32_t n_band = sh.counter;
          if (n_band <= kBandCap) {
            if (n_band > 0) pol.rescore_all(sh.cand_key, sh.cand_pos, n_band, qs, band);
          } else {
            all = true;  // a wide band: every candidate is rescored
          }
          __syncthreads();  // the counter and the band list are read above
        }
        if (all) pol.rescore_all(sh.cand_key, sh.cand_pos, n_cand, qs);
        __syncthreads();
      }
    }

    // 3. exact k-th largest key and the count above it (with too many
    //    candidates, the keys of the whole row are streamed -- computed exactly
    //    on the fly for certified rows)
    uint32_t T, above;
    const uint32_t n_src = overflow ? G : n_cand;
    if (overflow) {
      radix_kth_largest(FullKeys<P>{&pol}, G, (uint32_t)k, sh, &T, &above);
    } else if (compacted) {
      // the candidates share the bits that tau and the row's largest key share
      const int known = tau == top ? 32 : __clz(tau ^ top);
      radix_kth_largest(LdsCands{sh.cand_key}, n_cand, (uint32_t)k, sh, &T, &above, top, known,
                        32 - known);
    } else {
      radix_kth_largest(LdsCands{sh.cand_key}, n_cand, (uint32_t)k, sh, &T, &above);
    }
    const uint32_t need = (uint32_t)k - above;  // keys equal to T to keep, lowest positions first

    // 4. ordered keep pass: 4 consecutive entries per thread per round
    uint32_t out_base = 0, eq_base = 0;
    for (uint32_t base = 0; base < n_src; base += 4u * NT) {
      const uint32_t i0 = base + 4u * tid;
      uint32_t key[4], pos[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t i = i0 + e;
        if (i < n_src) {
          key[e] = overflow ? pol.full_key(i) : sh.cand_key[i];
          pos[e] = overflow ? i : sh.cand_pos[i];
        } else {
          key[e] = 0u;
          pos[e] = 0u;
        }
      }
      uint32_t eq_flags = 0, gt_flags = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (i0 + e < n_src) {
          eq_flags |= (key[e] == T ? 1u : 0u) << e;
          gt_flags |= (key[e] > T ? 1u : 0u) << e;
        }
      }
      // one scan of both counts (equal in the high half, above in the low
      // half; a round holds at most 4*NT entries, so neither half overflows)
      uint32_t both_tot;
      const uint32_t both = block_exclusive_sum<NT>(
          ((uint32_t)__popc(eq_flags) << 16) | (uint32_t)__popc(gt_flags), sh.wave_tot, &both_tot);
      const uint32_t eq_before = both >> 16, gt_before = both & 0xFFFFu;
      const uint32_t eq_tot = both_tot >> 16, gt_tot = both_tot & 0xFFFFu;
      // equal keys still to keep in this round, lowest positions first
      const uint32_t rem = need > eq_base ? need - eq_base : 0u;
      uint32_t eq_rank = eq_before;
      uint32_t o = out_base + gt_before + (eq_before < rem ? eq_before : rem);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool eq = (eq_flags >> e) & 1u;
        const bool keep = ((gt_flags >> e) & 1u) || (eq && eq_rank < rem);
        eq_rank += eq ? 1u : 0u;
        if (keep) em.keep(o++, pos[e]);
      }
      out_base += gt_tot + (eq_tot < rem ? eq_tot : rem);
      eq_base += eq_tot;
    }
    kept = out_base;  // == k
  }

  // 5. raw tail, width and padding
  if (ids) {
    const int32_t body = 4 * (int32_t)kept;
    const int32_t w = body + rv.tail;
    for (int i = body + tid; i < stride; i += NT)
      ids[i] = (i < w) ? (int32_t)(4 * rv.g + (i - body)) : -1;
  }
  if (width && tid == 0) width[row] = 4 * (int32_t)kept + rv.tail;
}

__global__ void __launch_bounds__(NT)
select_kernel(const float* __restrict__ scores, const uint32_t* __restrict__ maxima,
              const int32_t* __restrict__ seq_len, int32_t queries, int64_t g_max, int32_t k,
              int64_t row0, uint32_t* __restrict__ bitmap, int32_t* __restrict__ token_ids,
              int32_t* __restrict__ width) {
  __shared__ SelectShared sh;
  const int64_t lrow = blockIdx.x;
  const int64_t row = row0 + lrow;
  const RowView rv = row_view(seq_len, row, queries, g_max);
  const PlainScores pol{scores + lrow * g_max};
  select_row(pol, sh, scores, maxima, rv, lrow, row, g_max, k, bitmap, token_ids, width);
}

template <int HI, int DI>
__global__ void __launch_bounds__(NT)
select_certified_kernel(const float* __restrict__ scores, const uint32_t* __restrict__ maxima,
                        const int32_t* __restrict__ seq_len, int32_t queries, int64_t g_max,
                        int32_t k, int64_t row0, uint32_t* __restrict__ bitmap,
                        int32_t* __restrict__ token_ids, int32_t* __restrict__ width,
                        const float* __restrict__ index_q, const float* __restrict__ pooled,
                        const int64_t* __restrict__ pooled_off,
                        const float* __restrict__ widths) {
  __shared__ SelectShared sh;
  const int64_t lrow = blockIdx.x;
  const int64_t row = row0 + lrow;
  const RowView rv = row_view(seq_len, row, queries, g_max);
  const CertifiedScores<HI, DI> pol{index_q + row * (int64_t)(HI * DI),
                                    pooled + (rv.valid ? pooled_off[rv.b] : 0),
                                    widths ? widths + lrow * (g_max / 64) : nullptr};
  select_row(pol, sh, scores, maxima, rv, lrow, row, g_max, k, bitmap, token_ids, width);
}

// Bitmap -> chronological token IDs: popcount prefix over the words in order.
__global__ void __launch_bounds__(NT)
emit_kernel(const uint32_t* __restrict__ bitmap, const int32_t* __restrict__ seq_len,
            int32_t queries, int64_t g_max, int32_t k, int32_t* __restrict__ token_ids,
            int32_t* __restrict__ width) {
  __shared__ uint32_t wave_tot[NWAVES];
  const int tid = (int)threadIdx.x;
  const int64_t row = blockIdx.x;
  const RowView rv = row_view(seq_len, row, queries, g_max);
  const int32_t stride = 4 * k + 4;
  int32_t* ids = token_ids + row * stride;
  if (!rv.valid) {
    for (int i = tid; i < stride; i += NT) ids[i] = -1;
    if (tid == 0) width[row] = -1;
    return;
  }
  const uint32_t* bm = bitmap + row * (g_max / 32);
  const uint32_t G = (uint32_t)rv.g;
  const uint32_t words = (G + 31) / 32;
  uint32_t total = 0;
  for (uint32_t base = 0; base < words; base += 4u * NT) {
    const uint32_t w0 = base + 4u * tid;
    uint32_t wv[4];
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = w0 + e;
      uint32_t v = (w < words) ? bm[w] : 0u;
      if (w == words - 1 && (G & 31)) v &= (1u << (G & 31)) - 1u;  // bits past G
      wv[e] = v;
      cnt += (uint32_t)__popc(v);
    }
    uint32_t tot;
    uint32_t o = total + block_exclusive_sum<NT>(cnt, wave_tot, &tot);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t v = wv[e];
      while (v) {
        const uint32_t bit = (uint32_t)__ffs(v) - 1u;
        v &= v - 1u;
        if (o < (uint32_t)k) {
          const int32_t t = (int32_t)(4u * (32u * (w0 + e) + bit));
          *reinterpret_cast<int4*>(ids + 4 * o) = make_int4(t, t + 1, t + 2, t + 3);
        }
        ++o;
      }
    }
    total += tot;
  }
  __syncthreads();
  if (total > (uint32_t)k) {
    // more groups than the budget: not a selection this row can hold
    for (int i = tid; i < stride; i += NT) ids[i] = -1;
    if (tid == 0) width[row] = -1;
    return;
  }
  const int32_t body = 4 * (int32_t)total;
  const int32_t w = body + rv.tail;
  for (int i = body + tid; i < stride; i += NT)
    ids[i] = (i < w) ? (int32_t)(4 * rv.g + (i - body)) : -1;
  if (tid == 0) width[row] = w;
}

// The bounded dense row: every visible token 0..N-1 in order, for rows with
// at most 4k+3 visible tokens (AFN-017 §The dense-parity property: below the
// cut the sparse row is exactly this row; AFN-016 §Failure boundary: the
// dense oracle is bounded at 2,051 keys).  Longer or invalid rows get width -1.
__global__ void __launch_bounds__(256)
dense_ids_kernel(const int32_t* __restrict__ seq_len, int32_t queries, int32_t k,
                 int32_t* __restrict__ token_ids, int32_t* __restrict__ width) {
  const int64_t row = blockIdx.x;
  const int32_t stride = 4 * k + 4;
  const int32_t b = (int32_t)(row / queries);
  const int64_t n = (int64_t)seq_len[b] - queries + 1 + (row - (int64_t)b * queries);
  const bool ok = n >= 0 && n <= 4 * (int64_t)k + 3;
  int32_t* ids = token_ids + row * stride;
  for (int i = (int)threadIdx.x; i < stride; i += 256) ids[i] = (ok && i < n) ? i : -1;
  if (threadIdx.x == 0) width[row] = ok ? (int32_t)n : -1;
}

}  // namespace

int launch_dense_ids(const int32_t* seq_len, int32_t queries, int32_t k, int64_t rows,
                     int32_t* token_ids, int32_t* width, void* stream) {
  if (rows == 0) return 0;
  hipLaunchKernelGGL(dense_ids_kernel, dim3((unsigned)rows), dim3(256), 0,
                     static_cast<hipStream_t>(stream), seq_len, queries, k, token_ids, width);
  return hipGetLastError();
}

int launch_select(const SelectArgs& a, void* stream) {
  if (a.rows == 0) return 0;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)a.rows), dim3(NT), 0,
                     static_cast<hipStream_t>(stream), a.scores, a.maxima,
                     a.seq_len, a.queries, a.g_max, a.k, a.row0, a.bitmap, a.token_ids,
                     a.width);
  return hipGetLastError();
}

template <int HI, int DI>
hipError_t launch_cert_t(const SelectArgs& a, const RescoreArgs& r, hipStream_t s) {
  hipLaunchKernelGGL((select_certified_kernel<HI, DI>), dim3((unsigned)a.rows), dim3(NT), 0, s,
                     a.scores, a.maxima, a.seq_len, a.queries, a.g_max, a.k, a.row0, a.bitmap,
                     a.token_ids, a.width, r.index_q, r.pooled, r.pooled_off, a.widths);
  return hipGetLastError();
}

template <int HI>
hipError_t launch_cert_h(const SelectArgs& a, const RescoreArgs& r, hipStream_t s) {
  switch (r.index_dim) {
    case 32: return launch_cert_t<HI, 32>(a, r, s);
    case 64: return launch_cert_t<HI, 64>(a, r, s);
    case 128: return launch_cert_t<HI, 128>(a, r, s);
    default: return hipErrorInvalidValue;
  }
}

int launch_select_certified(const SelectArgs& a, const RescoreArgs& r, void* stream) {
  if (a.rows == 0) return 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (r.index_heads) {
    case 4: return launch_cert_h<4>(a, r, s);
    case 8: return launch_cert_h<8>(a, r, s);
    case 16: return launch_cert_h<16>(a, r, s);
    default: return hipErrorInvalidValue;
  }
}

int launch_emit(const uint32_t* bitmap, const int32_t* seq_len, int32_t queries, int64_t g_max,
                int32_t k, int64_t rows, int32_t* token_ids, int32_t* width, void* stream) {
  if (rows == 0) return 0;
  hipLaunchKernelGGL(emit_kernel, dim3((unsigned)rows), dim3(NT), 0,
                     static_cast<hipStream_t>(stream), bitmap, seq_len, queries, g_max, k,
                     token_ids, width);
  return hipGetLastError();
}

}  // namespace qsa
