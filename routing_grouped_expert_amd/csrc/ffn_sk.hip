// Grouped expert FFN: persistent kernels for the 16-byte fast path. The
// K-split kernels (one 16-token tile per pass: decode) and the staged
// kernels (4 or 8 token tiles per pass, token rows staged in LDS: prefill)
// share the schedule below.
//
// Why: the expert weights are streamed once and every config is HBM-bound, so
// the kernel time is (weight bytes) / (bandwidth actually sustained). A grid
// of equal blocks that does not divide evenly into the resident block slots
// leaves a last partial round with too few loads in flight. Here exactly the
// resident number of blocks NB is launched and the work is cut into units:
//   tile = (pass, row group)   pass = up to NT*16 tokens of one expert
//   unit = (tile, K chunk): K-split kernels 1024 (up; 512 when H is not a
//          multiple of 1024) or 512 (down), taken in two halves, the 4 waves
//          of a block taking a quarter of each half; staged kernels 64.
// Tiles are dealt in whole rounds; when the rounds come out uneven, the last
// tiles are cut into equal contiguous unit ranges (stream-K; see Sched).
// A block runs its units in order; the K-split kernels add their waves'
// partial sums in LDS in a fixed order (wave 0, 1, 2, 3) at the end of each
// tile. A tile covered by one block is finished directly; a tile cut between
// blocks leaves one partial per block in a slot, and the block that arrives
// last (atomic counter) adds the slots in block order and finishes the tile.
// The order of every sum is fixed by the schedule, so results do not depend
// on timing.
//
// Operands: weight rows are the MFMA A operand and stream from HBM into VGPRs
// as whole 128-byte lines (8 rows x 128 B per load instruction; bf16 weights
// then pass through a small wave-private LDS tile into fragment order, see
// slab_frags); the gathered token rows
// (page "FlashInfer MoE optimisation: overlapping grouped activation staging
// on Ampere and Hopper", flashinfer PR #7368, section 1: route index divided
// by the route divisor, 128-bit loads, absent members read as zero) are the B
// operand, loaded per lane from L2 with 16-byte loads. The loads of the next
// half unit are issued before the current half's MFMAs (section 2 of the same
// page: the weight stream starts first and overlaps the activation gather).
//
// up:   K-split tile rows = 16 gate rows + the 16 matching up rows; the
//       finished tile applies SwiGLU and writes a = silu(g) * u as
//       hi = bf16(a), lo = bf16(a - hi) (a is never rounded to bf16 alone).
// down: K-split tile rows = 128 rows of W2 (8 groups of 16 sharing each B
//       fragment); B = hi and lo, two MFMAs into one fp32 accumulator; the
//       finished tile writes fp32 expert_out.
#include "plan.h"

#include <algorithm>
#include <type_traits>

namespace moe {

int ffn_dense_blocks();
bool ffn_dense_shape_ok(int T, int k, int H, int I);
int ffn_dense_pass_tokens();
hipError_t launch_ffn_dense_up(const uint16_t* x, const int* perm, int k, int H, int I, int nmax,
                               const uint16_t* w1, const int* plan, int pmax, uint16_t* h_hi,
                               uint16_t* h_lo, hipStream_t stream);
hipError_t launch_ffn_dense_down(const uint16_t* h_hi, const uint16_t* h_lo, int k, int H, int I,
                                 int nmax, const uint16_t* w2, const int* plan, int pmax,
                                 float* out, hipStream_t stream);

namespace {
// Tile shapes, measured on MI355X at the decode shape (T32 H4096 I14336 E8
// top-2; up kernel / down kernel, microseconds). With fragment-layout weight
// loads:
//   up   1 gate group, 4 blocks per CU 354; 2 groups, 1 block per CU 320;
//        2 groups, 2 blocks 392; 4 groups, 1 block 354
//   down 8 groups, 1 block per CU 174; 4 groups 180-184; 16 groups 179;
//        the 4-group tiles of units of 4 steps, 2 blocks per CU 176
// With full-line slabs (two boxes):
//   up   2 groups x 2 steps 296-298; 1 group x 4 steps 269-271 (2 blocks per
//        CU 277); 1 x 8 270; 1 x 2, 2 blocks 279; 2 x 4 304
//   down 8 groups x 2 steps 147 / 166; 8 x 4 146 / 170; 4 x 2, 2 blocks 155;
//        4 x 4 158; 2 x 8 168
// A CU holding fewer weight rows open at once, each read in longer runs,
// streams faster; the token bytes per weight byte grow as the tile narrows
// but come from L2.
// MFMA K-steps (of 32) per wave per half unit; a unit is two halves, each
// spanning the 4 waves. The up projection takes 4 steps when H is a multiple
// of its 1024-wide unit, else 2.
constexpr int UP_STEPS = 4;
constexpr int UP_STEPS_SHORT = 2;
constexpr int DOWN_STEPS = 2;
constexpr int UP_KUNIT = 2 * 4 * 32 * UP_STEPS;
constexpr int UP_KUNIT_SHORT = 2 * 4 * 32 * UP_STEPS_SHORT;
constexpr int DOWN_KUNIT = 2 * 4 * 32 * DOWN_STEPS;
// Blocks per CU of the K-split kernels.
constexpr int UP_CAP = 1;
constexpr int DOWN_CAP = 1;
// FP8 weights: MFMA steps per half unit (even: a 16-byte load of codes feeds
// two steps) and blocks per CU (the up kernel at 3 blocks per CU, which its
// 100 VGPRs and 48 KB of LDS allow: 174 us against 169 us at 2, decode shape).
constexpr int UP8_STEPS = 4;
constexpr int DOWN8_STEPS = 4;
constexpr int UP8_KUNIT = 2 * 4 * 32 * UP8_STEPS;
constexpr int DOWN8_KUNIT = 2 * 4 * 32 * DOWN8_STEPS;
constexpr int UP8_CAP = 2;
constexpr int DOWN8_CAP = 1;
constexpr int UP_RG = 1;          // 16-row gate groups (and as many up groups) per up tile
constexpr int UP_ROWS = 16 * UP_RG;
// The FP8 up tile holds two gate groups (and two up groups): at one group the
// token fragments (bf16, 16 tokens) cost as many bytes per K step as the FP8
// weight codes, and the up kernel streamed slower (decode shape: 194 us
// against 167 us at two groups).
constexpr int UP8_RG = 2;
constexpr int UP8_ROWS = 16 * UP8_RG;
constexpr int DOWN_GROUPS = 8;    // 16-row groups per down tile
constexpr int DOWN_ROWS = 16 * DOWN_GROUPS;

// The plan (plan.h) lies at the start of the workspace; the fixup counters
// follow at a 256-byte boundary.

// Read-only view for the FFN kernels (the plan is written by an earlier
// kernel), so its wave-uniform entries are fetched with scalar loads.
struct PlanRO {
  const int* __restrict__ hdr;
  const int* __restrict__ expert;
  const int* __restrict__ beg;
  const int* __restrict__ cnt;
};

__device__ __forceinline__ PlanRO plan_ro(const int* __restrict__ plan, int pmax) {
  return PlanRO{plan, plan + 4, plan + 4 + pmax, plan + 4 + 2 * pmax};
}

// One block of 1024 threads: list the passes (expert, first entry, entries)
// of every local expert with entries, and zero the fixup counters.
__global__ __launch_bounds__(1024) void ffn_plan_kernel(const int* __restrict__ offsets, int L,
                                                        PlanOut po) {
  constexpr int nt = 1024;
  extern __shared__ __attribute__((aligned(16))) int s_lds[];  // 2 (L + 1) + 16
  int* off = s_lds;
  for (int i = threadIdx.x; i < po.ncounters; i += nt) po.counters[i] = 0;
  for (int i = threadIdx.x; i <= L; i += nt) off[i] = offsets[i];
  __syncthreads();
  write_ffn_plan(off, L, po, off + L + 1, nt);
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

// Full-line weight slabs (bf16 weights). Per row group a wave's weight
// operands for two MFMA K-steps are a slab of 16 rows x 64 elements (128
// bytes, one cache line per row). Loaded as MFMA fragments (lane l: row
// l % 16, 16 bytes), every load instruction reads half of each of 16 lines;
// loaded as two full-line loads (lane s: row s / 8, then 8 + s / 8, 16-byte
// chunk s % 8) with the nontemporal policy (every weight byte is read once),
// a plain stream of such slabs reads 6.6-7.0 TB/s on MI355X against 4.9-6.1
// TB/s. The wave then puts the slab in fragment order through a private 2 KB
// LDS tile: fragment st of lane l is chunk 4 st + l / 16 of row l % 16, the
// K order the token fragments already use. In the tile, chunk c of row r
// sits at slot c ^ (r % 8) of the row's 128 bytes, so both the writes and the
// reads spread over the LDS banks.
constexpr bool kFullLines = true;

// The lane's offset (elements) in a slab whose rows are ld elements apart;
// E elements make a 16-byte chunk (8 bf16, or 16 FP8 codes, whose slab spans
// the four MFMA steps of a 128-code line).
template <int E = 8>
__device__ __forceinline__ size_t slab_lane(int lane, size_t ld) {
  return (size_t)(lane >> 3) * ld + (lane & 7) * E;
}

// The two full-line loads (nontemporal) of the slab whose row 0, at the
// slab's K offset plus the lane's slab offset, is at p.
template <class V, class T>
__device__ __forceinline__ void slab_load(V (&v)[2], const T* p, size_t ld) {
  static_assert(sizeof(V) == 16, "16-byte chunks");
  v[0] = __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(p)));
  v[1] = __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(p + 8 * ld)));
}

// Slab -> the two MFMA fragments (16 bytes each), in place, through the
// wave's tile t (128 u16x8, private to the wave).
template <class V>
__device__ __forceinline__ void slab_frags(V (&v)[2], u16x8* t, int lane) {
  const int r0 = lane >> 3, c = lane & 7;
  t[r0 * 8 + (c ^ r0)] = __builtin_bit_cast(u16x8, v[0]);
  t[(8 + r0) * 8 + (c ^ r0)] = __builtin_bit_cast(u16x8, v[1]);
  const int r = lane & 15, g = lane >> 4, x = r & 7;
  v[0] = __builtin_bit_cast(V, t[r * 8 + (g ^ x)]);
  v[1] = __builtin_bit_cast(V, t[r * 8 + ((4 + g) ^ x)]);
}

// Block containing unit u when U units are cut into NB equal ranges
// [floor(b U / NB), floor((b + 1) U / NB)).
__device__ __forceinline__ int block_of_unit(long u, long U, int NB) {
  return (int)(((u + 1) * NB + U - 1) / U) - 1;
}
__device__ __forceinline__ long first_unit(int b, long U, int NB) { return (long)b * U / NB; }

// Position in a block's unit sequence: tile t, K chunk kc (unit t * C + kc).
// Tiles are numbered pass-major (t = pass * G + g) and fit in 32 bits; the
// main loops advance positions by additions only (a 64-bit division per step
// costs more than a step's arithmetic).
struct Pos {
  int t, kc;
};

// Chunk kc of a tile whose chunk order starts at `rot` (wrapping at C): a
// tile dealt whole to one block starts at chunk 7 tile % C, so the blocks
// streaming at the same moment read different offsets within their weight
// rows (see pf_issue); a tile cut between blocks keeps rot = 0, and so do the
// FP8 kernels (their code rows measured 1-2% slower rotated: fine-grained
// 2.289 against 2.248 ms, share 0 1.144 against 1.131 ms).
__device__ __forceinline__ int rot_chunk(int kc, int rot, int C) {
  const int c = kc + rot;
  return c >= C ? c - C : c;
}

// The units of a block. Tiles are dealt in whole rounds (in round r block b
// takes tile r NB + b, so the blocks running together on one XCD hold
// neighbouring tiles of the same pass and read its token rows from the same
// L2). When the rounds come out nearly even (TT >= 0.85 x rounds x NB) every
// tile is dealt whole and the last round simply has fewer blocks: the kernels
// are HBM-bound, so fewer blocks each stream faster. Otherwise R = TT / NB - 1
// whole rounds (none when TT < 2 NB) are followed by a stream-K share: the
// remaining tiles are cut into nb equal unit ranges, and a tile cut by a
// range boundary is finished through the cross-block fixup.
//
// Measured on the share-0 prefill shape (grouped FFN): stream-K over the last
// 1-2 rounds 2.03 ms, the same with one release per block and piece 1.68 ms,
// whole tiles only (4.8 and 8.4 rounds' work in 5 and 9 rounds) 1.64 ms.
struct Sched {
  int C, NB, TD, nb;
  long US;        // units of the stream-K part
  Pos ps, pe, p0; // the block's first and last stream-K unit, its first unit
  // A = 2: the stream-K cuts fall on even units only (C even), so a block's
  // units come in aligned pairs (the FP8 staged kernels load a pair's weight
  // codes as full lines); the fixup then counts in pairs (C / A, US / A).
  __device__ Sched(int b, int TT, int C_, int NB_, int A = 1) : C(C_), NB(NB_) {
    const int rounds = (TT + NB - 1) / NB;
    if ((long)TT * 100 >= (long)rounds * NB * 85) {
      TD = TT;
      US = 0;
      nb = min(TT, NB);
      const int lt = b < TT ? b + ((TT - 1 - b) / NB) * NB : 0;  // the block's last tile
      ps = pe = Pos{lt, C - 1};
      p0 = Pos{b, 0};
      return;
    }
    const int R = TT >= 2 * NB ? TT / NB - 1 : 0;
    TD = R * NB;
    US = (long)(TT - TD) * C;
    nb = (int)min((long)NB, US / A);
    const long s = A * first_unit(b, US / A, nb), e = A * first_unit(b + 1, US / A, nb) - 1;
    ps = Pos{TD + (int)(s / C), (int)(s % C)};
    pe = Pos{TD + (int)(e / C), (int)(e % C)};
    p0 = R > 0 ? Pos{b, 0} : ps;
  }
  __device__ bool last(Pos p) const { return p.t == pe.t && p.kc == pe.kc; }
  // the unit after p (p itself after the last)
  __device__ Pos next(Pos p) const {
    if (last(p)) return p;
    if (p.kc + 1 < C) return Pos{p.t, p.kc + 1};
    if (p.t >= TD) return Pos{p.t + 1, 0};
    return p.t + NB < TD ? Pos{p.t + NB, 0} : ps;
  }
  // the block's tile after t (t itself after the last)
  __device__ int next_tile(int t) const {
    if (t < TD) return t + NB < TD ? t + NB : ps.t;
    return t < pe.t ? t + 1 : pe.t;
  }
  __device__ bool ends_tile(Pos p) const { return p.kc == C - 1 || last(p); }
  // tile t is shared with another block
  __device__ bool split(int t) const {
    return t >= TD && ((t == ps.t && ps.kc > 0) || (t == pe.t && pe.kc < C - 1));
  }
};

// Sum the four waves' accumulators of one tile through LDS, RCH f32x4 per
// lane at a time: every wave writes its region, then wave 0 adds them in wave
// order 0, 1, 2, 3 into `acc`. Rounds alternate between two buffers
// (`parity`, carried from tile to tile), so a buffer is rewritten only after
// the next round's barrier, by which time wave 0 has read it. Every thread
// must call this.
constexpr int RCH = 4;
template <int N>
__device__ __forceinline__ void block_reduce(f32x4 (&acc)[N], f32x4 (*red)[4][RCH][kWave],
                                             int& parity, int wave, int lane) {
  static_assert(N % RCH == 0 || N < RCH, "rounds");
  constexpr int W = N < RCH ? N : RCH;
#pragma unroll
  for (int r = 0; r < N; r += W) {
#pragma unroll
    for (int i = 0; i < W; ++i) red[parity][wave][i][lane] = acc[r + i];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < W; ++i)
        acc[r + i] = ((red[parity][0][i][lane] + red[parity][1][i][lane]) + red[parity][2][i][lane]) +
                     red[parity][3][i][lane];
    }
    parity ^= 1;
  }
}

// Cross-block fixup of a tile cut between blocks. Each block stores its
// partial tile (`part`, N f32x4 per lane, per wave) into its slot; the block
// that arrives last (atomic counter) adds all slots in block order into
// `part`. A block holds at most two cut tiles (its first and its last): slot
// 2b for the first, 2b + 1 for the last; with SUBS waves taking part, wave w
// of a block uses sub-slot w.
//
// The device-scope fences that publish and receive the slots write back and
// invalidate the whole L2 of an XCD, which every block on it feels, so the
// release is issued once per block and piece, and the acquire only by the
// block that finishes the tile.
__device__ __forceinline__ int fixup_slot(int b, long t0, long U, int NB) {
  return 2 * b + (first_unit(b, U, NB) < t0 ? 1 : 0);
}

// One wave fixes up its block's piece (the K-split kernels: wave 0 after the
// in-block reduction).
template <int N>
__device__ bool fixup(f32x4 (&part)[N], f32x4* slots, int* counters, long tile, long C, long U,
                      int NB, int b, int lane) {
  const long t0 = tile * C;
  const int bf = block_of_unit(t0, U, NB), bl = block_of_unit(t0 + C - 1, U, NB);
  f32x4* mine = slots + (size_t)fixup_slot(b, t0, U, NB) * N * kWave;
#pragma unroll
  for (int i = 0; i < N; ++i) mine[i * kWave + lane] = part[i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  int last = 0;
  if (lane == 0) last = atomicAdd(&counters[bf], 1) == (bl - bf);
  last = __shfl(last, 0, kWave);
  if (!last) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
  for (int i = 0; i < N; ++i) part[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int pb = bf; pb <= bl; ++pb) {
    const f32x4* src = slots + (size_t)fixup_slot(pb, t0, U, NB) * N * kWave;
#pragma unroll
    for (int i = 0; i < N; ++i) part[i] = part[i] + src[i * kWave + lane];
  }
  return true;
}

// Every wave of the block holds its own part of the tile (the staged
// kernels): all SUBS waves store, the block meets, thread 0 publishes and
// counts, and if this block is the last, receives for the block. `flag` is an
// int in shared memory. Every thread must call this.
template <int N, int SUBS>
__device__ bool fixup_block(f32x4 (&part)[N], f32x4* slots, int* counters, long tile, long C,
                            long U, int NB, int b, int lane, int wave, int* flag) {
  const long t0 = tile * C;
  const int bf = block_of_unit(t0, U, NB), bl = block_of_unit(t0 + C - 1, U, NB);
  f32x4* mine = slots + ((size_t)fixup_slot(b, t0, U, NB) * SUBS + wave) * N * kWave;
#pragma unroll
  for (int i = 0; i < N; ++i) mine[i * kWave + lane] = part[i];
  // Every wave waits for its stores to reach L2 (vmcnt(0); the block barrier
  // alone does not wait for global stores), so thread 0's release, which
  // writes L2 back, covers the whole block's slot.
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int last = atomicAdd(&counters[bf], 1) == (bl - bf);
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *flag = last;
  }
  __syncthreads();
  if (!*flag) return false;
#pragma unroll
  for (int i = 0; i < N; ++i) part[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int pb = bf; pb <= bl; ++pb) {
    const f32x4* src = slots + ((size_t)fixup_slot(pb, t0, U, NB) * SUBS + wave) * N * kWave;
#pragma unroll
    for (int i = 0; i < N; ++i) part[i] = part[i] + src[i * kWave + lane];
  }
  return true;
}

// ----------------------------------------------------------------- up
// A tile is RG groups of 16 gate rows and the RG matching groups of up rows,
// all multiplied by the same token fragment: the token bytes a wave loads per
// weight byte are 1 / (2 RG), and on this chip the token loads share each
// CU's vector-memory path with the weight stream.
//
// Every token slot of the 16 is multiplied whatever the pass's entry count:
// columns past the entries are never stored. A branch on the count inside the
// main loop costs far more than the idle MFMAs: where the paths merge the
// compiler cannot tell whether the skipped operands' loads have landed, and
// waits for the next loads before issuing the ones after.

// Operands of one half unit for one wave (up projection).
template <int RG, int S>
struct UpOps {
  bf16x8 g[RG][S], u[RG][S], x[S];
  bool xz;  // the lane's entry is out of range: its token fragment reads as zero
};

// Loads go out row group by row group, so a lane's requests to one weight
// row follow each other (on the down projection at the decode shape this
// order took 176 us against 199 us for the groups interleaved step by step).
// With full-line slabs (S = 2) g / u hold the slabs until up_mma turns them
// into fragments.
template <int RG, int S>
__device__ __forceinline__ void up_load(UpOps<RG, S>& r, const uint16_t* wg, const uint16_t* wu,
                                        const uint16_t* x, int H, size_t kb, bool xz) {
  r.xz = xz;
  if constexpr (kFullLines) {
    static_assert(S % 2 == 0, "a slab is two MFMA steps");
#pragma unroll
    for (int q = 0; q < RG; ++q)
#pragma unroll
      for (int j = 0; j < S / 2; ++j)
        slab_load(*reinterpret_cast<bf16x8(*)[2]>(&r.g[q][2 * j]), wg + (size_t)q * 16 * H + kb + 64 * j, H);
#pragma unroll
    for (int q = 0; q < RG; ++q)
#pragma unroll
      for (int j = 0; j < S / 2; ++j)
        slab_load(*reinterpret_cast<bf16x8(*)[2]>(&r.u[q][2 * j]), wu + (size_t)q * 16 * H + kb + 64 * j, H);
  } else {
#pragma unroll
    for (int q = 0; q < RG; ++q)
#pragma unroll
      for (int st = 0; st < S; ++st) r.g[q][st] = ld8(wg + (size_t)q * 16 * H + kb + 32 * st);
#pragma unroll
    for (int q = 0; q < RG; ++q)
#pragma unroll
      for (int st = 0; st < S; ++st) r.u[q][st] = ld8(wu + (size_t)q * 16 * H + kb + 32 * st);
  }
#pragma unroll
  for (int st = 0; st < S; ++st) r.x[st] = ld8(x + kb + 32 * st);
}

// acc[q]: gate group q, acc[RG + q]: up group q. t: the wave's LDS tiles
// (RG S of 128 u16x8) for the full-line slabs.
template <int RG, int S>
__device__ __forceinline__ void up_mma(UpOps<RG, S>& r, f32x4 (&acc)[2 * RG], u16x8* t, int lane) {
#pragma unroll
  for (int st = 0; st < S; ++st) r.x[st] = r.xz ? bf16x8{} : r.x[st];
  if constexpr (kFullLines) {
#pragma unroll
    for (int q = 0; q < RG; ++q)
#pragma unroll
      for (int j = 0; j < S / 2; ++j) {
        slab_frags(*reinterpret_cast<bf16x8(*)[2]>(&r.g[q][2 * j]), t + ((2 * q) * (S / 2) + j) * 128, lane);
        slab_frags(*reinterpret_cast<bf16x8(*)[2]>(&r.u[q][2 * j]), t + ((2 * q + 1) * (S / 2) + j) * 128, lane);
      }
  }
#pragma unroll
  for (int st = 0; st < S; ++st)
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.g[q][st], r.x[st], acc[q], 0, 0, 0);
      acc[RG + q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.u[q][st], r.x[st], acc[RG + q], 0, 0, 0);
    }
}

// FP8 E4M3 weights (8-bit codes, one fp32 scale per row, applied to the
// finished sums): in a half unit a lane loads 16 codes per weight row, the K
// values of two MFMA steps: 16 (lane / 16) + 0..15 of each 64-wide piece of
// its wave's range, codes 0..7 for the even step and 8..15 for the odd one.
// The token fragments are loaded in the same K order, so the sum over K is
// unchanged; codes are widened to bf16 exactly just before their MFMAs.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int RG, int S>
struct UpOps8 {
  static_assert(S % 2 == 0, "pairs of MFMA steps");
  u32x4 g[RG][S / 2], u[RG][S / 2];
  bf16x8 x[S];
  bool xz;  // as in UpOps
};

template <int RG, int S>
__device__ __forceinline__ void up_load(UpOps8<RG, S>& r, const uint8_t* wg, const uint8_t* wu,
                                        const uint16_t* x, int H, size_t kb, bool xz) {
  r.xz = xz;
  if constexpr (kFullLines) {
    static_assert(S == 4, "an FP8 slab is four MFMA steps");
#pragma unroll
    for (int q = 0; q < RG; ++q) slab_load(r.g[q], wg + (size_t)q * 16 * H + kb, H);
#pragma unroll
    for (int q = 0; q < RG; ++q) slab_load(r.u[q], wu + (size_t)q * 16 * H + kb, H);
  } else {
#pragma unroll
    for (int q = 0; q < RG; ++q)
#pragma unroll
      for (int p = 0; p < S / 2; ++p)
        r.g[q][p] = *reinterpret_cast<const u32x4*>(wg + (size_t)q * 16 * H + kb + 64 * p);
#pragma unroll
    for (int q = 0; q < RG; ++q)
#pragma unroll
      for (int p = 0; p < S / 2; ++p)
        r.u[q][p] = *reinterpret_cast<const u32x4*>(wu + (size_t)q * 16 * H + kb + 64 * p);
  }
#pragma unroll
  for (int st = 0; st < S; ++st) r.x[st] = ld8(x + kb + 64 * (st / 2) + 8 * (st % 2));
}

template <int RG, int S>
__device__ __forceinline__ void up_mma(UpOps8<RG, S>& r, f32x4 (&acc)[2 * RG], u16x8* t, int lane) {
#pragma unroll
  for (int st = 0; st < S; ++st) r.x[st] = r.xz ? bf16x8{} : r.x[st];
  if constexpr (kFullLines) {
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      slab_frags(r.g[q], t + (2 * q) * 128, lane);
      slab_frags(r.u[q], t + (2 * q + 1) * 128, lane);
    }
  }
#pragma unroll
  for (int p = 0; p < S / 2; ++p)
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      const bf16x8 g0 = e4m3x8_to_bf16(r.g[q][p][0], r.g[q][p][1]);
      const bf16x8 g1 = e4m3x8_to_bf16(r.g[q][p][2], r.g[q][p][3]);
      const bf16x8 u0 = e4m3x8_to_bf16(r.u[q][p][0], r.u[q][p][1]);
      const bf16x8 u1 = e4m3x8_to_bf16(r.u[q][p][2], r.u[q][p][3]);
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g0, r.x[2 * p], acc[q], 0, 0, 0);
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g1, r.x[2 * p + 1], acc[q], 0, 0, 0);
      acc[RG + q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(u0, r.x[2 * p], acc[RG + q], 0, 0, 0);
      acc[RG + q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(u1, r.x[2 * p + 1], acc[RG + q], 0, 0, 0);
    }
}

// Per-tile state of the up projection, in two stages: `issue` loads the plan
// entries and the permutation row of a tile early (one tile ahead); `finish`
// turns them into addresses when the tile is reached, so those loads never
// stall the weight stream.
struct UpRaw {
  int g, ex, tb, tc, r, rot;
};
struct UpTile {
  int g, ex, tb, tc, rot;
  size_t wrow;  // lane's gate row (+ its K offset) in W1
  size_t xoff;  // lane's token row (+ its K offset) in x
  bool xz;      // the lane's entry is outside [0, T k): a zero row
};

__device__ __forceinline__ void up_issue(UpRaw& raw, int tile, int G, const PlanRO& pv,
                                         const int* perm, int lane, int C, int TD) {
  const int pass = tile / G;
  raw.rot = tile < TD ? (tile * 7) % C : 0;
  raw.g = tile - pass * G;
  raw.ex = pv.expert[pass];
  raw.tb = pv.beg[pass];
  raw.tc = pv.cnt[pass];
  const int n = lane & 15;
  raw.r = perm[raw.tb + (n < raw.tc ? n : 0)];
}

// Token slots past the pass's entries read a valid row (the first entry's):
// MFMA output column n depends only on B column n and those columns are never
// stored, so every load of the main loop is unconditional. An entry whose
// expanded index is outside [0, T k) reads token 0's row, and its fragment is
// replaced by zeros before the MFMAs (a zero row, as the interface states).
template <int RG>
__device__ __forceinline__ void up_finish(UpTile& st, const UpRaw& raw, int k, int H, int I,
                                          int nmax, size_t wlane, int kq) {
  st.g = raw.g;
  st.ex = raw.ex;
  st.tb = raw.tb;
  st.tc = raw.tc;
  st.rot = raw.rot;
  st.wrow = ((size_t)raw.ex * 2 * I + raw.g * (16 * RG)) * H + wlane;
  st.xz = !(raw.r >= 0 && raw.r < nmax);
  const int r = st.xz ? 0 : raw.r;
  st.xoff = (size_t)(r / k) * H + kq;
}

template <int RG, int S, bool F8>
__global__ __launch_bounds__(256) void ffn_up_sk_kernel(
    const uint16_t* __restrict__ x, const int* __restrict__ perm, int k, int H, int I, int nmax,
    const void* __restrict__ w1v, const float* __restrict__ s1, const int* __restrict__ plan,
    int pmax, f32x4* slots, int* counters, uint16_t* __restrict__ h_hi,
    uint16_t* __restrict__ h_lo, int NB) {
  constexpr int KHALF = 4 * 32 * S, KUNIT = 2 * KHALF, N = 2 * RG;
  using WT = std::conditional_t<F8, uint8_t, uint16_t>;
  using Ops = std::conditional_t<F8, UpOps8<RG, S>, UpOps<RG, S>>;
  const WT* w1 = static_cast<const WT*>(w1v);
  __shared__ f32x4 red[2][4][RCH][kWave];
  constexpr bool FL = kFullLines;
  constexpr int NSLAB = F8 ? 2 * RG : RG * S;  // slab tiles per wave
  __shared__ u16x8 slab_t[FL ? 4 : 1][FL ? NSLAB * 128 : 1];
  const PlanRO pv = plan_ro(plan, pmax);
  const int P = pv.hdr[0];
  const int G = I / (16 * RG), C = H / KUNIT;
  const int b = xcd_block(blockIdx.x, NB);
  const Sched rg(b, P * G, C, NB);
  if (b >= rg.nb) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int kq = (lane >> 4) * (F8 ? 16 : 8) + wave * 32 * S;
  // lane's offset from a row group's first row in W1
  const size_t wlane = FL ? slab_lane<F8 ? 16 : 8>(lane, H) + wave * 32 * S
                          : (size_t)(lane & 15) * H + kq;
  u16x8* tw = slab_t[FL ? wave : 0];
  const size_t I_H = (size_t)I * H;

  UpTile ts, tn;
  UpRaw rn;
  {
    UpRaw r0;
    up_issue(r0, rg.p0.t, G, pv, perm, lane, C, F8 ? 0 : rg.TD);
    up_finish<RG>(ts, r0, k, H, I, nmax, wlane, kq);
  }
  up_issue(rn, rg.next_tile(rg.p0.t), G, pv, perm, lane, C, F8 ? 0 : rg.TD);
  __builtin_amdgcn_sched_barrier(0);  // ahead of the weight loads

  f32x4 acc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // End of the tile of unit u: add the waves' partials, complete the tile
  // (directly, or through the cross-block fixup) and write a = silu(g) * u.
  int parity = 0;
  auto tile_end = [&](int tile) {
    block_reduce(acc, red, parity, wave, lane);
    if (wave == 0) {
      bool done = true;
      if (rg.split(tile)) done = fixup(acc, slots, counters, tile - rg.TD, C, rg.US, rg.nb, b, lane);
      const int n = lane & 15;
      if (done && n < ts.tc) {
        // lane l: rows 16 q + 4 (l / 16) + j of the tile, token slot l % 16
        typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int q = 0; q < RG; ++q) {
          u16x4 hi, lo;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float gg = acc[q][j], uu = acc[RG + q][j];
            if (F8) {
              const size_t row = (size_t)ts.ex * 2 * I + ts.g * (16 * RG) + q * 16 + (lane >> 4) * 4 + j;
              gg *= s1[row];
              uu *= s1[row + I];
            }
            const float a = gg / (1.0f + expf(-gg)) * uu;
            hi[j] = f32_to_bf16_bits(a);
            lo[j] = f32_to_bf16_bits(a - bf16_bits_to_f32(hi[j]));
          }
          const size_t o = (size_t)(ts.tb + n) * I + ts.g * (16 * RG) + q * 16 + (lane >> 4) * 4;
          *reinterpret_cast<u16x4*>(h_hi + o) = hi;
          *reinterpret_cast<u16x4*>(h_lo + o) = lo;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // One unit in two halves with their own registers: load the second half,
  // multiply the first; load the first half of the next unit (in the next
  // tile when this unit ends one), multiply the second; finish the tile when
  // this is its last unit in the block. Every unit starts with its first
  // half in flight in `h0`, so no register changes role between units.
  Ops h0, h1;
  up_load(h0, w1 + ts.wrow, w1 + ts.wrow + I_H, x + ts.xoff, H,
          (size_t)rot_chunk(rg.p0.kc, ts.rot, C) * KUNIT, ts.xz);
  __builtin_amdgcn_sched_barrier(0);
  for (Pos p = rg.p0;;) {
    up_load(h1, w1 + ts.wrow, w1 + ts.wrow + I_H, x + ts.xoff, H,
            (size_t)rot_chunk(p.kc, ts.rot, C) * KUNIT + KHALF, ts.xz);
    __builtin_amdgcn_sched_barrier(0);
    up_mma(h0, acc, tw, lane);
    const Pos pn = rg.next(p);  // past the end: p again (loaded, unused)
    if (pn.t != p.t) {
      up_finish<RG>(tn, rn, k, H, I, nmax, wlane, kq);
      up_issue(rn, rg.next_tile(pn.t), G, pv, perm, lane, C, F8 ? 0 : rg.TD);  // the tile after
    } else {
      tn = ts;
    }
    up_load(h0, w1 + tn.wrow, w1 + tn.wrow + I_H, x + tn.xoff, H,
            (size_t)rot_chunk(pn.kc, tn.rot, C) * KUNIT, tn.xz);
    __builtin_amdgcn_sched_barrier(0);
    up_mma(h1, acc, tw, lane);
    if (rg.ends_tile(p)) tile_end(p.t);
    if (rg.last(p)) break;
    ts = tn;
    p = pn;
  }
}

// --------------------------------------------------------------- down
// A tile is DG groups of 16 rows of W2 sharing each B fragment (hi and lo of
// the intermediate: two MFMAs into one fp32 accumulator).

// Operands of one half unit for one wave (down projection).
template <int DG, int S>
struct DownOps {
  bf16x8 a[DG][S], h[S], l[S];
};

template <int DG, int S>
__device__ __forceinline__ void down_load(DownOps<DG, S>& r, const uint16_t* w, int I,
                                          const uint16_t* hh, const uint16_t* hl, size_t kb) {
  if constexpr (kFullLines) {
    static_assert(S % 2 == 0, "a slab is two MFMA steps");
#pragma unroll
    for (int q = 0; q < DG; ++q)
#pragma unroll
      for (int j = 0; j < S / 2; ++j)
        slab_load(*reinterpret_cast<bf16x8(*)[2]>(&r.a[q][2 * j]), w + (size_t)q * 16 * I + kb + 64 * j, I);
  } else {
#pragma unroll
    for (int q = 0; q < DG; ++q)
#pragma unroll
      for (int st = 0; st < S; ++st) r.a[q][st] = ld8(w + (size_t)q * 16 * I + kb + 32 * st);
  }
#pragma unroll
  for (int st = 0; st < S; ++st) {
    r.h[st] = ld8(hh + kb + 32 * st);
    r.l[st] = ld8(hl + kb + 32 * st);
  }
}

// t: the wave's LDS tiles (DG S / 2 of 128 u16x8) for the full-line slabs.
template <int DG, int S>
__device__ __forceinline__ void down_mma(DownOps<DG, S>& r, f32x4 (&acc)[DG], u16x8* t, int lane) {
  if constexpr (kFullLines) {
#pragma unroll
    for (int q = 0; q < DG; ++q)
#pragma unroll
      for (int j = 0; j < S / 2; ++j)
        slab_frags(*reinterpret_cast<bf16x8(*)[2]>(&r.a[q][2 * j]), t + (q * (S / 2) + j) * 128, lane);
  }
#pragma unroll
  for (int st = 0; st < S; ++st)
#pragma unroll
    for (int q = 0; q < DG; ++q) {
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.a[q][st], r.h[st], acc[q], 0, 0, 0);
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.a[q][st], r.l[st], acc[q], 0, 0, 0);
    }
}

// FP8 weights for the down projection, with the K order of UpOps8.
template <int DG, int S>
struct DownOps8 {
  static_assert(S % 2 == 0, "pairs of MFMA steps");
  u32x4 a[DG][S / 2];
  bf16x8 h[S], l[S];
};

template <int DG, int S>
__device__ __forceinline__ void down_load(DownOps8<DG, S>& r, const uint8_t* w, int I,
                                          const uint16_t* hh, const uint16_t* hl, size_t kb) {
  if constexpr (kFullLines) {
    static_assert(S == 4, "an FP8 slab is four MFMA steps");
#pragma unroll
    for (int q = 0; q < DG; ++q) slab_load(r.a[q], w + (size_t)q * 16 * I + kb, I);
  } else {
#pragma unroll
    for (int q = 0; q < DG; ++q)
#pragma unroll
      for (int p = 0; p < S / 2; ++p)
        r.a[q][p] = *reinterpret_cast<const u32x4*>(w + (size_t)q * 16 * I + kb + 64 * p);
  }
#pragma unroll
  for (int st = 0; st < S; ++st) {
    r.h[st] = ld8(hh + kb + 64 * (st / 2) + 8 * (st % 2));
    r.l[st] = ld8(hl + kb + 64 * (st / 2) + 8 * (st % 2));
  }
}

template <int DG, int S>
__device__ __forceinline__ void down_mma(DownOps8<DG, S>& r, f32x4 (&acc)[DG], u16x8* t, int lane) {
  if constexpr (kFullLines) {
#pragma unroll
    for (int q = 0; q < DG; ++q) slab_frags(r.a[q], t + q * 128, lane);
  }
#pragma unroll
  for (int p = 0; p < S / 2; ++p)
#pragma unroll
    for (int q = 0; q < DG; ++q) {
      const bf16x8 a0 = e4m3x8_to_bf16(r.a[q][p][0], r.a[q][p][1]);
      const bf16x8 a1 = e4m3x8_to_bf16(r.a[q][p][2], r.a[q][p][3]);
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, r.h[2 * p], acc[q], 0, 0, 0);
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, r.l[2 * p], acc[q], 0, 0, 0);
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, r.h[2 * p + 1], acc[q], 0, 0, 0);
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, r.l[2 * p + 1], acc[q], 0, 0, 0);
    }
}

// Per-tile state of the down projection (plan entries loaded a tile ahead).
struct DownRaw {
  int g, ex, tb, tc, rot;
};
struct DownTile {
  int g, ex, tb, tc, rot;
  size_t wrow;  // lane's first W2 row (+ its K offset)
  size_t hrow;  // lane's row of h (+ its K offset)
};

__device__ __forceinline__ void down_issue(DownRaw& raw, int tile, int G, const PlanRO& pv, int C,
                                           int TD) {
  const int pass = tile / G;
  raw.rot = tile < TD ? (tile * 7) % C : 0;
  raw.g = tile - pass * G;
  raw.ex = pv.expert[pass];
  raw.tb = pv.beg[pass];
  raw.tc = pv.cnt[pass];
}

template <int DG>
__device__ __forceinline__ void down_finish(DownTile& st, const DownRaw& raw, int H, int I,
                                            int lane, size_t wlane, int kq) {
  st.g = raw.g;
  st.ex = raw.ex;
  st.tb = raw.tb;
  st.tc = raw.tc;
  st.rot = raw.rot;
  st.wrow = ((size_t)raw.ex * H + raw.g * (16 * DG)) * I + wlane;
  const int n = lane & 15;  // slots past the entries read the first entry's row
  st.hrow = (size_t)(raw.tb + (n < raw.tc ? n : 0)) * I + kq;
}

template <int DG, int S, bool F8>
__global__ __launch_bounds__(256) void ffn_down_sk_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int H, int I,
    const void* __restrict__ w2v, const float* __restrict__ s2, const int* __restrict__ plan,
    int pmax, f32x4* slots, int* counters, float* __restrict__ out, int NB) {
  constexpr int KHALF = 4 * 32 * S, KUNIT = 2 * KHALF;
  using WT = std::conditional_t<F8, uint8_t, uint16_t>;
  using Ops = std::conditional_t<F8, DownOps8<DG, S>, DownOps<DG, S>>;
  const WT* w2 = static_cast<const WT*>(w2v);
  __shared__ f32x4 red[2][4][RCH][kWave];
  constexpr bool FL = kFullLines;
  constexpr int NSLAB = F8 ? DG : DG * S / 2;  // slab tiles per wave
  __shared__ u16x8 slab_t[FL ? 4 : 1][FL ? NSLAB * 128 : 1];
  const PlanRO pv = plan_ro(plan, pmax);
  const int P = pv.hdr[0];
  const int G = H / (16 * DG), C = I / KUNIT;
  const int b = xcd_block(blockIdx.x, NB);
  const Sched rg(b, P * G, C, NB);
  if (b >= rg.nb) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int kq = (lane >> 4) * (F8 ? 16 : 8) + wave * 32 * S;
  // lane's offset from a row group's first row in W2
  const size_t wlane = FL ? slab_lane<F8 ? 16 : 8>(lane, I) + wave * 32 * S
                          : (size_t)(lane & 15) * I + kq;
  u16x8* tw = slab_t[FL ? wave : 0];

  DownTile ts, tn;
  DownRaw rn;
  {
    DownRaw r0;
    down_issue(r0, rg.p0.t, G, pv, C, F8 ? 0 : rg.TD);
    down_finish<DG>(ts, r0, H, I, lane, wlane, kq);
  }
  down_issue(rn, rg.next_tile(rg.p0.t), G, pv, C, F8 ? 0 : rg.TD);

  f32x4 acc[DG];
#pragma unroll
  for (int i = 0; i < DG; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  int parity = 0;
  auto tile_end = [&](int tile) {
    block_reduce(acc, red, parity, wave, lane);
    if (wave == 0) {
      bool done = true;
      if (rg.split(tile)) done = fixup(acc, slots, counters, tile - rg.TD, C, rg.US, rg.nb, b, lane);
      const int n = lane & 15;
      if (F8) {
#pragma unroll
        for (int q = 0; q < DG; ++q)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[q][j] *= s2[(size_t)ts.ex * H + ts.g * (16 * DG) + q * 16 + (lane >> 4) * 4 + j];
      }
      if (done && n < ts.tc) {
        float* o = out + (size_t)(ts.tb + n) * H + ts.g * (16 * DG) + (lane >> 4) * 4;
#pragma unroll
        for (int q = 0; q < DG; ++q) *reinterpret_cast<f32x4*>(o + q * 16) = acc[q];
      }
    }
#pragma unroll
    for (int i = 0; i < DG; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // Units in two halves, as in the up projection.
  Ops h0, h1;
  down_load(h0, w2 + ts.wrow, I, h_hi + ts.hrow, h_lo + ts.hrow,
            (size_t)rot_chunk(rg.p0.kc, ts.rot, C) * KUNIT);
  __builtin_amdgcn_sched_barrier(0);
  for (Pos p = rg.p0;;) {
    down_load(h1, w2 + ts.wrow, I, h_hi + ts.hrow, h_lo + ts.hrow,
              (size_t)rot_chunk(p.kc, ts.rot, C) * KUNIT + KHALF);
    __builtin_amdgcn_sched_barrier(0);
    down_mma(h0, acc, tw, lane);
    const Pos pn = rg.next(p);
    if (pn.t != p.t) {
      down_finish<DG>(tn, rn, H, I, lane, wlane, kq);
      down_issue(rn, rg.next_tile(pn.t), G, pv, C, F8 ? 0 : rg.TD);  // the tile after
    } else {
      tn = ts;
    }
    down_load(h0, w2 + tn.wrow, I, h_hi + tn.hrow, h_lo + tn.hrow,
              (size_t)rot_chunk(pn.kc, tn.rot, C) * KUNIT);
    __builtin_amdgcn_sched_barrier(0);
    down_mma(h1, acc, tw, lane);
    if (rg.ends_tile(p)) tile_end(p.t);
    if (rg.last(p)) break;
    ts = tn;
    p = pn;
  }
}

// ================================================================ prefill
// Many tokens per expert. A block of 8 waves owns a tile of 256 weight rows
// (32 per wave: two 16-row MFMA groups) and walks its K range in 64-wide
// chunks. The chunk of the pass's token rows (B operand, up to 128 tokens) is
// staged once per block in LDS and read by all 8 waves, so each token byte
// brought in serves 256 weight rows. Token rows are loaded two chunks ahead
// (registers, then one of two LDS buffers) and weights one chunk ahead (two
// for the up projection with 8 token tiles), so no wait in a step is for a
// load issued in the same step. Up tiles hold 128 gate rows and the matching
// 128 up rows (a wave: 16 of each), so SwiGLU is applied in the epilogue.
// bf16 weights arrive as one full-line slab per group and chunk; FP8 codes
// (16 per lane and group, fragment layout) are widened to bf16 just before
// the MFMAs and the row scales applied to the finished sums.
//
// Weights and token rows share a CU's vector-memory path: the token-row bytes
// per weight byte (tokens / tile rows, doubled for the hi + lo intermediate
// of the down projection) limit how close the weights stream comes to the
// HBM rate, hence the tall tiles; at the share-0 shape the MFMA phase of each
// chunk, which the weight loads one chunk ahead do not fully cover, costs
// more than the token traffic.
constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = PF_WAVES * kWave;
constexpr int PF_K = 64;
constexpr int PF_STEPS = PF_K / 32;
constexpr int PF_GROUPS = 2;                        // 16-row MFMA groups per wave
constexpr int PF_ROWS = PF_WAVES * 16 * PF_GROUPS;  // weight rows per tile
constexpr int PF_UP_COLS = PF_ROWS / 2;             // h columns per up tile

// A staged token row holds one 64-wide chunk (128 bytes, eight 16-byte
// pieces); piece q of row n sits at slot q ^ (n % 8), so both the stores of
// whole rows and the MFMA fragment reads (16 rows, one piece each, per 16
// lanes) run without LDS bank conflicts. Rows padded to 144 bytes instead
// took 4 conflict cycles per fragment read (a probe of such reads on MI355X:
// 270 against 495 B/ns per CU).
typedef uint16_t pf_row_t[PF_K];
__device__ __forceinline__ int pf_slot(int n, int q) { return ((q ^ n) & 7) * 8; }

// One 64-wide chunk of NR B rows: thread t holds pieces t, t + 512, ...
// (piece = row n, 16-byte column q).
template <int NR>
struct PfStage {
  static constexpr int PIECES = NR * (PF_K / 8);
  static constexpr int PER = (PIECES + PF_THREADS - 1) / PF_THREADS;
  u16x8 v[PER];
};

// Token rows are read through a buffer resource over the whole source array:
// the pieces of rows past the pass's entries carry an offset beyond the
// resource's size, which the hardware answers with zeros without a memory
// request, so padding costs no traffic and needs no branch.
constexpr uint32_t kPadOffset = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pf_rsrc(const uint16_t* base, size_t elems) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, (int)(elems * 2),
                                           0x00020000);
}

template <int NR>
__device__ __forceinline__ void pf_stage_load(PfStage<NR>& st, __amdgpu_buffer_rsrc_t rs,
                                              const uint32_t (&voff)[PfStage<NR>::PER],
                                              uint32_t kb_bytes) {
#pragma unroll
  for (int i = 0; i < PfStage<NR>::PER; ++i)
    st.v[i] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], kb_bytes, 0));
}

template <int NR>
__device__ __forceinline__ void pf_stage_store(const PfStage<NR>& st, pf_row_t* dst, int tid) {
#pragma unroll
  for (int i = 0; i < PfStage<NR>::PER; ++i) {
    const int piece = tid + PF_THREADS * i;
    if (PfStage<NR>::PIECES % PF_THREADS == 0 || piece < PfStage<NR>::PIECES)
      *reinterpret_cast<u16x8*>(&dst[piece / (PF_K / 8)][pf_slot(piece / (PF_K / 8), piece % (PF_K / 8))]) = st.v[i];
  }
}

// A lane's weight operands: bf16, one chunk, a full-line slab per group (two
// MFMA fragments once through the LDS tile); FP8, the aligned pair of chunks
// that one 128-code line per row spans, loaded as a full-line slab per group
// and put through the LDS tile into fragment layout: v[q][h] holds chunk h of
// the pair, lane l row l % 16, codes 16 (l / 16) .. + 15 of the 64-wide chunk
// (codes + 0..7 feed the first MFMA step, + 8..15 the second, and the token
// fragments are read in that K order).
template <bool F8>
struct PfA {
  bf16x8 v[PF_GROUPS][PF_STEPS];
};
template <>
struct PfA<true> {
  u32x4 v[PF_GROUPS][2];
};

// acc[q * NT + nt] += A(group q) * B(token tile nt) over one chunk for the
// first NV token tiles (the others hold no entry of the pass and keep zero
// sums); the down projection multiplies both halves (hi, lo) of the
// intermediate.
template <int NT, int NV, bool UP, bool F8>
__device__ __forceinline__ void pf_mma(const PfA<F8>& a, const pf_row_t* b0, const pf_row_t* b1,
                                       int lane, f32x4* acc, int nv, int half) {
#pragma unroll
  for (int st = 0; st < PF_STEPS; ++st) {
    bf16x8 w[PF_GROUPS];
#pragma unroll
    for (int q = 0; q < PF_GROUPS; ++q) {
      if constexpr (F8) {
        const u32x4& c = half ? a.v[q][1] : a.v[q][0];
        w[q] = e4m3x8_to_bf16(c[2 * st], c[2 * st + 1]);
      }
      else w[q] = a.v[q][st];
    }
#pragma unroll
    for (int nt = 0; nt < NV; ++nt) {
      if (nt >= nv) break;
      const int n = nt * 16 + (lane & 15);
      const int c = F8 ? (lane >> 4) * 16 + st * 8 : st * 32 + (lane >> 4) * 8;
      const bf16x8 h = *reinterpret_cast<const bf16x8*>(&b0[n][pf_slot(n, c / 8)]);
#pragma unroll
      for (int q = 0; q < PF_GROUPS; ++q)
        acc[q * NT + nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[q], h, acc[q * NT + nt], 0, 0, 0);
      if (!UP) {
        const bf16x8 l = *reinterpret_cast<const bf16x8*>(&b1[n][pf_slot(n, c / 8)]);
#pragma unroll
        for (int q = 0; q < PF_GROUPS; ++q)
          acc[q * NT + nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[q], l, acc[q * NT + nt], 0, 0, 0);
      }
    }
  }
}

// Tile state (plan entries and the B rows' offsets), loaded a tile ahead.
template <int NT>
struct PfRaw {
  int g, ex, tb, tc, rot;
  int r[PfStage<NT * 16>::PER];
};

// A tile dealt whole to one block walks its K chunks starting at chunk
// 7 tile % C (wrapping round; rot_chunk), so the blocks streaming at the same
// moment read different offsets within their weight rows. Rows whose length
// is a multiple of 4 KB otherwise put every block's current 128 bytes at the
// same low address bits: the down projection at I = 2048 (4 KB rows) read
// 5.1 TB/s against 5.7 TB/s at I = 1920 and 2176, and rotating took the
// fine-grained FFN from 3.65 to 3.51 ms and share 0 from 1.41 to 1.36 ms
// (starting at 7 tile % C rather than tile % C: 1.34 ms at share 0). A tile
// cut between blocks (stream-K) is not rotated.
template <int NT, bool UP>
__device__ __forceinline__ void pf_issue(PfRaw<NT>& raw, int tile, int G, const PlanRO& pv,
                                         const int* perm, int tid, int C, int TD) {
  const int pass = tile / G;
  raw.rot = tile < TD ? (tile * 7) % C : 0;
  raw.g = tile - pass * G;
  raw.ex = pv.expert[pass];
  raw.tb = pv.beg[pass];
  raw.tc = pv.cnt[pass];
#pragma unroll
  for (int i = 0; i < PfStage<NT * 16>::PER; ++i) {
    const int n = (tid + PF_THREADS * i) / (PF_K / 8);
    const int nn = n < raw.tc ? n : 0;  // rows past the entries read the first entry's row
    raw.r[i] = UP ? perm[raw.tb + nn] : raw.tb + nn;
  }
}

template <int NT>
struct PfTile {
  int g, ex, tb, tc, ntiles, rot;
  size_t wrow;                               // this lane's first weight row (+ K offset)
  uint32_t voff[PfStage<NT * 16>::PER];      // staged B rows (+ this thread's column), bytes
};

// Weight row of group q relative to the lane's first row: up groups 0, 1 are
// gate rows c0 .. c0 + 31 and groups 2, 3 the up rows I + c0 .. ; down groups
// are 16 consecutive output rows each.
template <bool UP>
__device__ __forceinline__ size_t pf_group_offset(int q, int H, int I) {
  constexpr int HALF = PF_GROUPS / 2;
  return UP ? (size_t)((q % HALF) * 16 + (q / HALF) * I) * H : (size_t)q * 16 * I;
}

template <int NT, bool UP, bool F8>
__device__ __forceinline__ void pf_finish(PfTile<NT>& st, const PfRaw<NT>& raw, int k, int H,
                                          int I, int nmax, int wave, int lane, int tid) {
  st.g = raw.g;
  st.ex = raw.ex;
  st.tb = raw.tb;
  st.tc = raw.tc;
  st.ntiles = (raw.tc + 15) >> 4;
  st.rot = raw.rot;
  const int kq = (lane >> 4) * 8;
  const int K = UP ? H : I;
  const int row = UP ? raw.g * PF_UP_COLS + wave * 8 * PF_GROUPS
                     : raw.g * PF_ROWS + wave * 16 * PF_GROUPS;
  st.wrow = (UP ? ((size_t)raw.ex * 2 * I + row) : ((size_t)raw.ex * H + row)) * K +
            (F8 ? slab_lane<16>(lane, K)
                : (kFullLines ? slab_lane(lane, K) : (size_t)(lane & 15) * K + kq));
#pragma unroll
  for (int i = 0; i < PfStage<NT * 16>::PER; ++i) {
    const int n = (tid + PF_THREADS * i) / (PF_K / 8), q = (tid + PF_THREADS * i) % (PF_K / 8);
    int r = raw.r[i];
    bool ok = n < raw.tc;
    if (UP) {  // an expanded index outside [0, T k) gathers a zero row
      ok = ok && r >= 0 && r < nmax;
      r = ok ? r / k : 0;
    }
    st.voff[i] = ok ? (uint32_t)((r * K + q * 8) * 2) : kPadOffset;
  }
}

// The up projection with 4 token tiles is held to 128 VGPRs, so that two
// blocks share a CU. The down projection with 4 token tiles runs one block
// per CU with its weights two chunks ahead (146 VGPRs): fine-grained FFN
// 3.635 against 3.682 ms for two blocks per CU one chunk ahead (two blocks
// and two chunks ahead spill at 128 VGPRs: 4.10 ms).
// F8: FP8 E4M3 weight codes with one fp32 scale per row (wscale), applied to
// the finished sums.
template <int NT, bool UP, bool F8>
__global__ __launch_bounds__(PF_THREADS, (NT <= 4 && UP) ? 4 : 1) void ffn_pf_kernel(
    const uint16_t* __restrict__ b0src, const uint16_t* __restrict__ b1src,
    const int* __restrict__ perm, int k, int H, int I, int nmax, const void* __restrict__ wv,
    const float* __restrict__ wscale, const int* __restrict__ plan, int pmax, f32x4* slots,
    int* counters, uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo,
    float* __restrict__ out, int NB) {
  using WT = std::conditional_t<F8, uint8_t, uint16_t>;
  const WT* w = static_cast<const WT*>(wv);
  constexpr bool FL = kFullLines && !F8;  // bf16 slabs through the wave's LDS tile
  constexpr bool SLAB = FL || F8;          // FP8: pair slabs through the same tile
  constexpr int NR = NT * 16;
  constexpr int NACC = PF_GROUPS * NT;
  constexpr int NB_ARR = UP ? 1 : 2;  // B arrays: x, or h_hi and h_lo
  __shared__ __attribute__((aligned(16))) pf_row_t bs[2][NB_ARR][NR];
  __shared__ u16x8 slab_t[SLAB ? PF_WAVES : 1][SLAB ? PF_GROUPS * 128 : 1];
  __shared__ int fix_flag;
  const PlanRO pv = plan_ro(plan, pmax);
  if (pv.hdr[1] != 0) return;  // the dense kernels take this plan
  const int P = pv.hdr[0];
  const int K = UP ? H : I;
  const int G = UP ? I / PF_UP_COLS : H / PF_ROWS, C = K / PF_K;
  const int b = xcd_block(blockIdx.x, NB);
  constexpr int A = F8 ? 2 : 1;  // FP8: units in aligned pairs (C is even)
  const Sched sc(b, P * G, C, NB, A);
  if (b >= sc.nb) return;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const Pos p0 = sc.p0;
  // token rows: x (T = nmax / k rows of H) or h_hi and h_lo (nmax rows of I)
  const __amdgpu_buffer_rsrc_t rs0 = pf_rsrc(b0src, UP ? (size_t)(nmax / k) * H : (size_t)nmax * I);
  const __amdgpu_buffer_rsrc_t rs1 = pf_rsrc(b1src, (size_t)nmax * I);

  // Tile states of the units in the pipeline: t0 for chunk p (multiplied this
  // step), t1 for chunk p1 (its weights are loaded this step, its token rows
  // were loaded the step before), t2 for chunk p2 (its token rows are loaded
  // this step); rn holds the plan entries of the tile after t2's.
  PfTile<NT> t0, t1, t2;
  PfRaw<NT> rn;
  Pos p1 = sc.next(p0);
  {
    PfRaw<NT> r0;
    pf_issue<NT, UP>(r0, p0.t, G, pv, perm, tid, C, F8 ? 0 : sc.TD);
    pf_finish<NT, UP, F8>(t0, r0, k, H, I, nmax, wave, lane, tid);
    if (p1.t != p0.t) {
      pf_issue<NT, UP>(r0, p1.t, G, pv, perm, tid, C, F8 ? 0 : sc.TD);
      pf_finish<NT, UP, F8>(t1, r0, k, H, I, nmax, wave, lane, tid);
    } else {
      t1 = t0;
    }
  }
  pf_issue<NT, UP>(rn, sc.next_tile(p1.t), G, pv, perm, tid, C, F8 ? 0 : sc.TD);

  f32x4 acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto chunk = [&](const PfTile<NT>& t, int kc) {  // the tile's kc-th chunk (rotated)
    return (size_t)rot_chunk(kc, t.rot, C) * PF_K;
  };
  auto load_a = [&](PfA<F8>& a, const PfTile<NT>& t, int kc) {
    if constexpr (F8) {  // the pair holding chunk kc (FP8 tiles are not rotated)
      const size_t kb = (size_t)(kc & ~1) * PF_K;
#pragma unroll
      for (int q = 0; q < PF_GROUPS; ++q) slab_load(a.v[q], w + t.wrow + pf_group_offset<UP>(q, H, I) + kb, K);
      return;
    }
    const size_t kb = chunk(t, kc);
    if constexpr (kFullLines) {
      static_assert(PF_STEPS == 2, "a slab is two MFMA steps");
#pragma unroll
      for (int q = 0; q < PF_GROUPS; ++q)
        slab_load(a.v[q], w + t.wrow + pf_group_offset<UP>(q, H, I) + kb, K);
    } else {
#pragma unroll
      for (int q = 0; q < PF_GROUPS; ++q)
#pragma unroll
        for (int st = 0; st < PF_STEPS; ++st)
          a.v[q][st] = ld8(w + t.wrow + pf_group_offset<UP>(q, H, I) + kb + 32 * st);
    }
  };
  auto load_b = [&](PfStage<NR> (&st)[NB_ARR], const PfTile<NT>& t, int kc) {
    const size_t kb = chunk(t, kc);
    pf_stage_load(st[0], rs0, t.voff, (uint32_t)(kb * 2));
    if (!UP) pf_stage_load(st[NB_ARR - 1], rs1, t.voff, (uint32_t)(kb * 2));
  };
  auto store_b = [&](const PfStage<NR> (&st)[NB_ARR], int buf) {
    pf_stage_store(st[0], bs[buf][0], tid);
    if (!UP) pf_stage_store(st[NB_ARR - 1], bs[buf][NB_ARR - 1], tid);
  };

  // End of tile p.t in this block: complete it (directly, or through the
  // cross-block fixup when the stream-K cut falls inside it) and write it.
  auto tile_end = [&](Pos p) {
    bool done = true;
    if (sc.split(p.t))
      done = fixup_block<NACC, PF_WAVES>(acc, slots, counters, p.t - sc.TD, C / A, sc.US / A, sc.nb, b,
                                         lane, wave, &fix_flag);
    if (done) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = nt * 16 + (lane & 15);
        if (n >= t0.tc) continue;
        if (UP) {
          typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
          for (int q = 0; q < PF_GROUPS / 2; ++q) {
            u16x4 hi, lo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float gg = acc[q * NT + nt][j], uu = acc[(q + PF_GROUPS / 2) * NT + nt][j];
              if constexpr (F8) {
                const size_t row = (size_t)t0.ex * 2 * I + t0.g * PF_UP_COLS +
                                   wave * 8 * PF_GROUPS + q * 16 + (lane >> 4) * 4 + j;
                gg *= wscale[row];
                uu *= wscale[row + I];
              }
              const float a = gg / (1.0f + expf(-gg)) * uu;
              hi[j] = f32_to_bf16_bits(a);
              lo[j] = f32_to_bf16_bits(a - bf16_bits_to_f32(hi[j]));
            }
            const int col = t0.g * PF_UP_COLS + wave * 8 * PF_GROUPS + q * 16 + (lane >> 4) * 4;
            const size_t o = (size_t)(t0.tb + n) * I + col;
            *reinterpret_cast<u16x4*>(h_hi + o) = hi;
            *reinterpret_cast<u16x4*>(h_lo + o) = lo;
          }
        } else {
#pragma unroll
          for (int q = 0; q < PF_GROUPS; ++q) {
            const int row = t0.g * PF_ROWS + wave * 16 * PF_GROUPS + q * 16 + (lane >> 4) * 4;
            f32x4 v = acc[q * NT + nt];
            if constexpr (F8) {
#pragma unroll
              for (int j = 0; j < 4; ++j) v[j] *= wscale[(size_t)t0.ex * H + row + j];
            }
            *reinterpret_cast<f32x4*>(out + (size_t)(t0.tb + n) * H + row) = v;
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // prologue: chunk p0's token rows in LDS buffer 0 and its weights in
  // registers; chunk p1's token rows in flight
  // A3: the up projection with 8 token tiles (238 VGPRs) fetches its weights
  // two units ahead, through three register sets (share 0: 882 us against
  // 911 us one unit ahead), and so does the down projection with 4 token
  // tiles (one block per CU, see the launch bounds); the bf16 down projection
  // at 8 tiles measured the same either way and stays at one unit ahead.
  // FP8: two register sets, each the full-line slab of a pair of units,
  // fetched at the pair's first unit for the pair two units ahead.
  constexpr bool A3 = !F8 && ((UP && NT >= 8) || (!UP && NT == 4));
  PfA<F8> a0, a1, a2;  // a2: A3 only
  PfStage<NR> sb0[NB_ARR], sb1[NB_ARR];
  load_b(sb1, t0, p0.kc);
  load_a(a0, t0, p0.kc);
  if constexpr (A3) load_a(a1, t1, p1.kc);
  store_b(sb1, 0);
  load_b(sb0, t1, p1.kc);
  __syncthreads();

  // One unit: issue chunk p2's token rows and chunk p1's (A3: p2's; FP8 at a
  // pair's first unit: the pair p2 starts) weights, multiply chunk p (weights
  // `ca`, half `half` of an FP8 pair; token rows in LDS buffer `cb`), write
  // chunk p1's token rows (`cs`, loaded a step earlier) into the other
  // buffer, finish the tile if p ends it here, and synchronise the block.
  // Returns false after the block's last unit.
  auto step = [&](int half, PfA<F8>& ca, PfA<F8>& na, PfStage<NR> (&cs)[NB_ARR],
                  PfStage<NR> (&ns)[NB_ARR], int cb, Pos& p) -> bool {
    const Pos p2 = sc.next(p1);
    if (p2.t != p1.t) {
      pf_finish<NT, UP, F8>(t2, rn, k, H, I, nmax, wave, lane, tid);
      pf_issue<NT, UP>(rn, sc.next_tile(p2.t), G, pv, perm, tid, C, F8 ? 0 : sc.TD);
    } else {
      t2 = t1;
    }
    load_b(ns, t2, p2.kc);
    if constexpr (F8) {
      if (half == 0) load_a(na, t2, p2.kc);  // (after the last pair: its own again)
    } else if constexpr (A3) {
      load_a(na, t2, p2.kc);
    } else {
      load_a(na, t1, p1.kc);
    }
    if (FL || (F8 && half == 0)) {
#pragma unroll
      for (int q = 0; q < PF_GROUPS; ++q) slab_frags(ca.v[q], slab_t[wave] + q * 128, lane);
    }
    // Token tiles of the pass that hold entries; the MFMAs and LDS reads of
    // the others are skipped (their sums stay zero). Passes are often far
    // from full: at the fine-grained shape 1 or 2 of 4 tiles, at share 0
    // 4 to 7 of 8 (share 0: 1.42 ms against 1.52-1.56 ms for the call). The
    // test sits inside the tile loop: dispatching to kernels unrolled for
    // fewer tiles made every variant spill.
    const int nv = __builtin_amdgcn_readfirstlane(t0.ntiles);
    pf_mma<NT, NT, UP, F8>(ca, bs[cb][0], bs[cb][NB_ARR - 1], lane, acc, nv, half);
    store_b(cs, cb ^ 1);
    const bool last = sc.last(p);
    if (sc.ends_tile(p)) tile_end(p);
    __syncthreads();
    if (last) return false;
    t0 = t1;
    t1 = t2;
    p = p1;
    p1 = p2;
    return true;
  };

  constexpr int h0 = 0, h1 = 1;
  Pos p = p0;
  if constexpr (F8) {
    while (step(h0, a0, a1, sb0, sb1, 0, p) && step(h1, a0, a1, sb1, sb0, 1, p) &&
           step(h0, a1, a0, sb0, sb1, 0, p) && step(h1, a1, a0, sb1, sb0, 1, p)) {
    }
  } else if constexpr (A3) {
    while (step(h0, a0, a2, sb0, sb1, 0, p) && step(h0, a1, a0, sb1, sb0, 1, p) &&
           step(h0, a2, a1, sb0, sb1, 0, p) && step(h0, a0, a2, sb1, sb0, 1, p) &&
           step(h0, a1, a0, sb0, sb1, 0, p) && step(h0, a2, a1, sb1, sb0, 1, p)) {
    }
  } else {
    while (step(h0, a0, a1, sb0, sb1, 0, p) && step(h0, a1, a0, sb1, sb0, 1, p)) {
    }
  }
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Resident blocks of `threads` threads of kernel K on the current device
// (cached per kernel and device).
template <auto K>
int resident_blocks(int threads = 256, int cap = 8) {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, threads, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    if (per_cu > cap) per_cu = cap;  // at most 8: the workspace holds slots for 8 blocks per CU
    cached[dev] = per_cu * device_cus();
  }
  return cached[dev];
}

// Token tiles (of 16) per pass, from twice the mean entries per local expert
// (an expert with more entries takes further passes, each reading its weights
// again), capped by T (a token picks an expert at most once). 1: the K-split
// kernels; 4 or 8: the kernels with token rows staged in LDS. With 8, the
// dense kernels (ffn_dense.hip: passes of 256 tokens, both operands staged in
// LDS) may take the call instead, which the plan writer decides from the
// local entry counts (at least kDenseMean per local expert). Between 16 and 32 the staged kernels with 4 tiles
// win over 2-tile passes: on the fine-grained shape (T512 H7168 I2048 E256
// top-8) 4.05 ms against 5.46 ms, mostly by not repeating passes for the
// experts above 32 entries. Staged kernels at 2 tiles (weights two chunks
// ahead, at most 120 VGPRs) took the same shape's grouped FFN to 3.79 ms
// against 3.69 ms at 4 tiles.
constexpr int kDenseMean = 112;
int pick_nt(int T, int k, int L) {
  const long bound = T;
  const long twice_mean = L > 0 ? (2L * T * k + L - 1) / L : bound;
  const long want = twice_mean < bound ? twice_mean : bound;
  return want <= 16 ? 1 : want <= 64 ? 4 : 8;
}
// Whether the dense kernels may take the call: the local entries can reach
// kDenseMean per local expert (T k of them at most), the shape suits them,
// bf16 weights. The plan writer then decides from the actual counts.
bool dense_possible(int T, int k, int L, int H, int I, bool f8) {
  return !f8 && L > 0 && (long)T * k >= (long)kDenseMean * L && pick_nt(T, k, L) == 8 &&
         ffn_dense_shape_ok(T, k, H, I);
}

size_t a256(size_t n) { return (n + 255) & ~(size_t)255; }

template <int NT>
int up_blocks(bool f8) {
  if constexpr (NT == 1)
    return f8 ? resident_blocks<ffn_up_sk_kernel<UP8_RG, UP8_STEPS, true>>(256, UP8_CAP)
              : std::min(resident_blocks<ffn_up_sk_kernel<UP_RG, UP_STEPS, false>>(256, UP_CAP),
                         resident_blocks<ffn_up_sk_kernel<UP_RG, UP_STEPS_SHORT, false>>(256, UP_CAP));
  else
    return f8 ? resident_blocks<ffn_pf_kernel<NT, true, true>>(PF_THREADS)
              : resident_blocks<ffn_pf_kernel<NT, true, false>>(PF_THREADS);
}
template <int NT>
int down_blocks(bool f8) {
  if constexpr (NT == 1)
    return f8 ? resident_blocks<ffn_down_sk_kernel<DOWN_GROUPS, DOWN8_STEPS, true>>(256, DOWN8_CAP)
              : resident_blocks<ffn_down_sk_kernel<DOWN_GROUPS, DOWN_STEPS, false>>(256, DOWN_CAP);
  else
    return f8 ? resident_blocks<ffn_pf_kernel<NT, false, true>>(PF_THREADS)
              : resident_blocks<ffn_pf_kernel<NT, false, false>>(PF_THREADS);
}

int blocks_for(int NT, bool up, bool f8) {
  switch (NT) {
    case 1: return up ? up_blocks<1>(f8) : down_blocks<1>(f8);
    case 4: return up ? up_blocks<4>(f8) : down_blocks<4>(f8);
    default: return up ? up_blocks<8>(f8) : down_blocks<8>(f8);
  }
}

// Workspace after h_hi / h_lo: the plan, then per kernel (up, down) `subs`
// counters per block, and 2 x `subs` slots per block shared by both kernels
// (a block's first and last tile; `subs` = 1 for the K-split kernels, one per
// wave for the prefill kernels). A slot holds one wave's partial tile: for the
// K-split kernels the largest of the tiles' accumulators (2 UP_RG, 2 UP8_RG or
// DOWN_GROUPS f32x4 per lane), for the prefill kernels at most 4 NT.
struct SkLayout {
  size_t plan, counters, slots, total;
  int pmax, nb_up, nb_down, subs;
};

SkLayout sk_layout(int T, int k, int L, int NT, bool f8) {
  SkLayout o{};
  const int nmax = T * k, nr = NT * 16;
  o.pmax = L + (nmax + nr - 1) / nr + 1;
  o.nb_up = blocks_for(NT, true, f8);
  o.nb_down = blocks_for(NT, false, f8);
  const int nbm = o.nb_up > o.nb_down ? o.nb_up : o.nb_down;
  o.plan = 0;
  o.subs = NT == 1 ? 1 : PF_WAVES;
  o.counters = a256((size_t)(4 + kPlanArrays * o.pmax) * 4);
  o.slots = o.counters + a256((size_t)2 * o.subs * nbm * 4);
  const int slot_n = NT == 1 ? std::max({2 * UP_RG, 2 * UP8_RG, DOWN_GROUPS}) : 4 * NT;
  o.total = o.slots + a256((size_t)2 * o.subs * nbm * slot_n * kWave * 16);
  return o;
}

// dense: the dense kernels may take the call (the plan writer decides).
PlanOut plan_out(const SkLayout& lo, char* ws, int T, int k, int NT, bool dense) {
  const int nbm = lo.nb_up > lo.nb_down ? lo.nb_up : lo.nb_down;
  return PlanOut{reinterpret_cast<int*>(ws + lo.plan), lo.pmax, NT * 16, T * k,
                 reinterpret_cast<int*>(ws + lo.counters), 2 * lo.subs * nbm,
                 dense ? ffn_dense_pass_tokens() : 0, kDenseMean};
}

// plan_ready: the plan and zeroed counters are already in the workspace
// (written by the routing's permutation kernel), so no plan kernel runs.
template <int NT>
hipError_t launch_sk_nt(const uint16_t* x, const int* perm, const int* offsets, int L, int T,
                        int k, int H, int I, const void* w1, const void* w2, const float* s1,
                        const float* s2, uint16_t* h_hi, uint16_t* h_lo, float* out, char* ws,
                        bool plan_ready, hipStream_t stream) {
  // s1 / s2 non-null: FP8 weight codes with row scales
  const bool f8 = s1 != nullptr;
  const SkLayout lo = sk_layout(T, k, L, NT, f8);
  const bool dense = NT == 8 && dense_possible(T, k, L, H, I, f8);
  const PlanOut po = plan_out(lo, ws, T, k, NT, dense);
  int* plan = po.plan;
  int* counters = po.counters;
  f32x4* slots = reinterpret_cast<f32x4*>(ws + lo.slots);
  const int nmax = T * k;
  const int nbm = lo.nb_up > lo.nb_down ? lo.nb_up : lo.nb_down;
  hipError_t err = hipSuccess;
  if (!plan_ready) {
    hipLaunchKernelGGL(ffn_plan_kernel, dim3(1), dim3(1024), (size_t)(2 * (L + 1) + 16) * 4,
                       stream, offsets, L, po);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if constexpr (NT == 1) {
    if (f8)
      hipLaunchKernelGGL((ffn_up_sk_kernel<UP8_RG, UP8_STEPS, true>), dim3(lo.nb_up), dim3(256), 0,
                         stream, x, perm, k, H, I, nmax, w1, s1, plan, lo.pmax, slots, counters,
                         h_hi, h_lo, lo.nb_up);
    else if (H % UP_KUNIT == 0)
      hipLaunchKernelGGL((ffn_up_sk_kernel<UP_RG, UP_STEPS, false>), dim3(lo.nb_up), dim3(256), 0,
                         stream, x, perm, k, H, I, nmax, w1, s1, plan, lo.pmax, slots, counters,
                         h_hi, h_lo, lo.nb_up);
    else
      hipLaunchKernelGGL((ffn_up_sk_kernel<UP_RG, UP_STEPS_SHORT, false>), dim3(lo.nb_up),
                         dim3(256), 0, stream, x, perm, k, H, I, nmax, w1, s1, plan, lo.pmax,
                         slots, counters, h_hi, h_lo, lo.nb_up);
  } else {
    if (f8)
      hipLaunchKernelGGL((ffn_pf_kernel<NT, true, true>), dim3(lo.nb_up), dim3(PF_THREADS), 0,
                         stream, x, x, perm, k, H, I, nmax, w1, s1, plan, lo.pmax, slots,
                         counters, h_hi, h_lo, out, lo.nb_up);
    else
      hipLaunchKernelGGL((ffn_pf_kernel<NT, true, false>), dim3(lo.nb_up), dim3(PF_THREADS), 0,
                         stream, x, x, perm, k, H, I, nmax, w1, s1, plan, lo.pmax, slots,
                         counters, h_hi, h_lo, out, lo.nb_up);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // The dense kernels' turn when the plan writer chose them (the staged
  // kernels then return at once, and the other way round).
  if (dense) {
    err = launch_ffn_dense_up(x, perm, k, H, I, nmax, static_cast<const uint16_t*>(w1), plan,
                              lo.pmax, h_hi, h_lo, stream);
    if (err != hipSuccess) return err;
  }
  if constexpr (NT == 1) {
    if (f8)
      hipLaunchKernelGGL((ffn_down_sk_kernel<DOWN_GROUPS, DOWN8_STEPS, true>), dim3(lo.nb_down),
                         dim3(256), 0, stream, h_hi, h_lo, H, I, w2, s2, plan, lo.pmax, slots,
                         counters + lo.subs * nbm, out, lo.nb_down);
    else
      hipLaunchKernelGGL((ffn_down_sk_kernel<DOWN_GROUPS, DOWN_STEPS, false>), dim3(lo.nb_down),
                         dim3(256), 0, stream, h_hi, h_lo, H, I, w2, s2, plan, lo.pmax, slots,
                         counters + lo.subs * nbm, out, lo.nb_down);
  } else {
    if (f8)
      hipLaunchKernelGGL((ffn_pf_kernel<NT, false, true>), dim3(lo.nb_down), dim3(PF_THREADS), 0,
                         stream, h_hi, h_lo, perm, k, H, I, nmax, w2, s2, plan, lo.pmax, slots,
                         counters + lo.subs * nbm, h_hi, h_lo, out, lo.nb_down);
    else
      hipLaunchKernelGGL((ffn_pf_kernel<NT, false, false>), dim3(lo.nb_down), dim3(PF_THREADS), 0,
                         stream, h_hi, h_lo, perm, k, H, I, nmax, w2, s2, plan, lo.pmax, slots,
                         counters + lo.subs * nbm, h_hi, h_lo, out, lo.nb_down);
  }
  err = hipGetLastError();
  if (err != hipSuccess || !dense) return err;
  return launch_ffn_dense_down(h_hi, h_lo, k, H, I, nmax, static_cast<const uint16_t*>(w2), plan,
                               lo.pmax, out, stream);
}
}  // namespace

bool ffn_sk_applies(const void* x, const void* w1, const void* w2, const void* out, int T, int k,
                    int L, int H, int I) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (!(al(x) && al(w1) && al(w2) && al(out))) return false;
  if (pick_nt(T, k, L) == 1)
    return H % UP_KUNIT_SHORT == 0 && I % DOWN_KUNIT == 0 && I % UP_ROWS == 0 &&
           H % DOWN_ROWS == 0;
  // the staged kernels address token rows with 32-bit byte offsets below 2^31
  const size_t lim = (size_t)1 << 31;
  return H % PF_K == 0 && I % PF_K == 0 && H % PF_ROWS == 0 && I % PF_UP_COLS == 0 &&
         (size_t)T * H * 2 < lim && (size_t)T * k * I * 2 < lim;
}

// The plan the persistent kernels will read for these sizes, in the FFN's own
// workspace `ws` (the part after h_hi / h_lo), for a caller that writes it
// itself.
PlanOut ffn_sk_plan_out(int T, int k, int L, int H, int I, bool f8, void* ws) {
  const int nt = pick_nt(T, k, L);
  return plan_out(sk_layout(T, k, L, nt, f8), static_cast<char*>(ws), T, k, nt,
                  nt == 8 && dense_possible(T, k, L, H, I, f8));
}

// The dense kernels read only the plan, which the staged layout holds (its
// passes of 128 entries outnumber passes of 256).
size_t ffn_sk_workspace_bytes(int T, int k, int L) {
  const int nt = pick_nt(T, k, L);
  const size_t a = sk_layout(T, k, L, nt, false).total;
  const size_t b = sk_layout(T, k, L, nt, true).total;  // the FP8 kernels' share of it
  return a > b ? a : b;
}

hipError_t launch_grouped_ffn_sk(const uint16_t* x, const int* perm, const int* offsets, int L,
                                 int T, int k, int H, int I, const uint16_t* w1,
                                 const uint16_t* w2, uint16_t* h_hi, uint16_t* h_lo, float* out,
                                 void* ws, bool plan_ready, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  switch (pick_nt(T, k, L)) {
    case 1: return launch_sk_nt<1>(x, perm, offsets, L, T, k, H, I, w1, w2, nullptr, nullptr, h_hi, h_lo, out, w, plan_ready, stream);
    case 4: return launch_sk_nt<4>(x, perm, offsets, L, T, k, H, I, w1, w2, nullptr, nullptr, h_hi, h_lo, out, w, plan_ready, stream);
    default: return launch_sk_nt<8>(x, perm, offsets, L, T, k, H, I, w1, w2, nullptr, nullptr, h_hi, h_lo, out, w, plan_ready, stream);
  }
}

// FP8 weights (codes + row scales) on the persistent kernels (K-split or
// staged, by the entries per expert): shapes for which ffn_sk_fp8_applies
// holds.
bool ffn_sk_fp8_applies(const void* x, const void* w1q, const void* w2q, const void* out, int T,
                        int k, int L, int H, int I) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (!(al(x) && al(w1q) && al(w2q) && al(out))) return false;
  if (pick_nt(T, k, L) == 1)
    return H % UP8_KUNIT == 0 && I % DOWN8_KUNIT == 0 && I % UP8_ROWS == 0 && H % DOWN_ROWS == 0;
  // the staged kernels address token rows with 32-bit byte offsets below 2^31
  const size_t lim = (size_t)1 << 31;
  return H % PF_K == 0 && I % PF_K == 0 && H % PF_ROWS == 0 && I % PF_UP_COLS == 0 &&
         (size_t)T * H * 2 < lim && (size_t)T * k * I * 2 < lim;
}

hipError_t launch_grouped_ffn_sk_fp8(const uint16_t* x, const int* perm, const int* offsets,
                                     int L, int T, int k, int H, int I, const uint8_t* w1q,
                                     const float* w1s, const uint8_t* w2q, const float* w2s,
                                     uint16_t* h_hi, uint16_t* h_lo, float* out, void* ws,
                                     bool plan_ready, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  switch (pick_nt(T, k, L)) {
    case 1: return launch_sk_nt<1>(x, perm, offsets, L, T, k, H, I, w1q, w2q, w1s, w2s, h_hi, h_lo, out, w, plan_ready, stream);
    case 4: return launch_sk_nt<4>(x, perm, offsets, L, T, k, H, I, w1q, w2q, w1s, w2s, h_hi, h_lo, out, w, plan_ready, stream);
    default: return launch_sk_nt<8>(x, perm, offsets, L, T, k, H, I, w1q, w2q, w1s, w2s, h_hi, h_lo, out, w, plan_ready, stream);
  }
}

}  // namespace moe
