// Grouped expert FFN for experts with many entries (prefill batches of
// thousands of tokens): the contraction is dense enough to be bound by the
// matrix cores rather than by the weight stream, so both operands are staged
// in LDS and every byte staged feeds a tall and wide tile.
//
// Page "FlashInfer MoE optimisation: overlapping grouped activation staging
// on Ampere and Hopper" (flashinfer PR #7368): section 1 (the routed rows of
// a group are gathered with 128-bit copies into on-chip memory, absent
// members read as zeros) and section 2 (the weight tile and the gathered
// activations are staged ahead of the matrix instructions, and a barrier
// publishes every stage before any wave reads it).
//
// Why a separate kernel: the staged kernels of ffn_sk.hip pair each weight
// tile with at most 128 tokens, which is 128 flop per weight byte; against
// the ~312 flop/byte ridge of 2.5 PFLOP/s over 8 TB/s an expert with
// hundreds of entries then stays bound by re-reading its weights once per
// 128 tokens. Here a tile is 256 weight rows x 256 tokens (256 flop per
// weight byte within the block, and passes of one expert that run together
// on an XCD share its weight lines in L2), computed by 8 waves of 128 rows x
// 64 tokens each (v_mfma_f32_16x16x32_bf16, fp32 accumulate; a wave quarter
// takes every fourth 16-token group, see dn_groups).
//
// Staging: each 32-wide K stage of both operands goes HBM/L2 -> LDS by
// buffer loads that write LDS directly (one 1 KB block of 16 rows x 64 bytes
// per wave instruction, no VGPR round trip; a probe of such loads from L2
// moved 120-145 B/ns per CU, as many as loads into VGPRs), several stages
// ahead (4 LDS stage slots for the up projection, 3 for the down projection,
// whose token operand is the hi and lo halves of the intermediate). Rows past a pass's
// entries carry a buffer offset beyond the resource, which reads zeros with
// no memory request. Within a block, 16-byte piece q of row r sits at slot
// q ^ ((r >> 1) & 3): the MFMA fragment reads (16 rows, one piece each, per
// 16 lanes) then run without bank conflicts. Measured on MI355X with a probe
// of such reads (16 waves per CU): 490 B/ns per CU conflict-free, against
// 280 B/ns and 4 conflict cycles per read for rows without the XOR, for
// rows padded to 144 bytes, for q ^ (r & 3) and for q ^ (((r >> 1) ^
// (r >> 3)) & 3).
//
// Pipeline: one block barrier per stage; stages run on across a block's
// tiles (its next tile starts loading while the current one finishes), and a
// tile's epilogue writes its outputs right after its last stage. The up
// projection reads the next stage's fragments (a second register set) while
// the MFMAs of the current one run; the down projection, whose hi + lo
// fragments leave no room for a second set, reads a stage's fragments at its
// start. The buffer-to-LDS loads are written as asm, so that the compiler
// does not track them: it cannot tell the stage slots apart across the loop
// and would otherwise wait for every load in flight before each LDS read. A
// stage is published by the kernel itself: each wave waits for its own loads
// of the stage (vmcnt), then the block meets.
//
// Tiles: 256 tokens per pass, numbered row tile first within an expert (see
// dn_tile), dealt round-robin over the resident blocks (one per CU),
// renumbered so that an XCD's blocks hold neighbouring tiles.
//
// Measured at the probe shape (share-0 expert weights, T32768: 52524 local
// entries, 4.63 TFLOP useful): up 3.42 ms, down 2.93 ms; grouped FFN 6.35 ms
// against 9.41 ms for the staged kernels (29% against 20% of the bf16 peak).
// Timing-only copies of the first version (up / down, ms): as built 3.44 /
// 2.94, loads and barriers only 2.78 / 1.92, MFMAs and barriers only 2.40 /
// 1.95: the load side (each stage waits for its slowest HBM miss, and the
// LDS holds only three stages of loads in flight) and the MFMA side (a
// barrier every 32 MFMAs per wave; the clock runs near 1.95 GHz under this
// load) each bound the kernel near 2.4-2.8 ms. Tiles numbered row tile first
// took the up kernel's HBM reads from 12.7 to 9.6 GB (L2 hits 81%).
//
// up:   tile = 128 h columns: rows 0-63 of wave half 0 are the gate rows of
//       the first 64 columns and rows 64-127 their up rows, likewise for wave
//       half 1; the epilogue applies SwiGLU and writes hi = bf16(a),
//       lo = bf16(a - hi), as the other grouped-FFN kernels do.
// down: tile = 256 output rows of W2; the token operand is hi and lo, two
//       MFMAs per fragment pair into one fp32 accumulator; fp32 expert_out.
#include "plan.h"

#include <algorithm>
#include <type_traits>

namespace moe {

namespace {

constexpr int DN_WAVES = 8;
constexpr int DN_THREADS = DN_WAVES * kWave;
constexpr int DN_ROWS = 256;             // weight rows per tile
constexpr int DN_TOK = 256;              // tokens per pass
constexpr int DN_K = 32;                 // K per stage
constexpr int DN_UP_COLS = DN_ROWS / 2;  // h columns per up tile
constexpr int DN_UP_STAGES = 4;
constexpr int DN_DOWN_STAGES = 3;
constexpr uint32_t kDnPad = 0x80000000u;  // a buffer offset past every resource


__device__ __forceinline__ int dn_swz(int r) { return (r >> 1) & 3; }

// Plan entries of tile t. The tiles of an expert's passes are numbered row
// tile first, pass second: with the expert's P passes starting at pass Q,
// its tiles are Q G .. (Q + P) G - 1 and tile Q G + i is row tile i / P of
// pass Q + i % P. The blocks running together on an XCD then hold all passes
// of a few weight tiles, which share those weight lines in L2, and tiles of
// one pass, which share its token rows.
struct DnTile {
  int t, ex, beg, cnt, g;
};

__device__ __forceinline__ DnTile dn_tile(const int* __restrict__ plan, int pmax, int t, int G) {
  const int q0 = t / G;
  const int first = plan[4 + 3 * pmax + q0], np = plan[4 + 4 * pmax + q0];
  const int i = t - first * G;
  const int g = i / np;
  const int pass = first + (i - g * np);
  DnTile d;
  d.t = t;
  d.g = g;
  d.ex = plan[4 + pass];
  d.beg = plan[4 + pmax + pass];
  d.cnt = plan[4 + 2 * pmax + pass];
  return d;
}

// A buffer resource (four SGPRs) over `bytes` bytes from `base`: offsets at
// or past `bytes` read zeros without a memory request.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 dn_rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// One 1 KB block (16 rows) of a stage, loaded by the whole wave straight into
// LDS at byte address `lds`: lane i fills slot i (row i / 4, slot i % 4).
// Written as asm so that the compiler does not track these LDS writes: it
// cannot tell the stage slots apart across the loop and would otherwise wait
// for every load in flight before each LDS read. The kernel publishes each
// stage itself (its wait for the wave's own loads, then the block barrier).
__device__ __forceinline__ void dn_dma(const u32x4& rs, uint32_t lds, uint32_t voff,
                                       uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
      : "memory", "m0");
}

// The loads a wave issues for one stage: blocks 2w and 2w + 1 of the weight
// tile and of the token tile (and of the lo half for the down projection).
struct DnIssue {
  u32x4 ra;               // the tile's expert matrix
  uint32_t va[2], vb[2];  // this lane's byte offsets in its two blocks
  int t, kc;              // tile and stage being issued
};

template <bool UP>
__device__ __forceinline__ void dn_issue_tile(DnIssue& is, const DnTile& d,
                                              const int* __restrict__ perm, const uint16_t* w,
                                              int k, int H, int I, int nmax, int wave, int lane) {
  const int K = UP ? H : I;
  const int r = lane >> 2, q = (lane & 3) ^ dn_swz(r);
  if (UP) {
    is.ra = dn_rsrc4(w + (size_t)d.ex * 2 * I * H, (uint32_t)((size_t)2 * I * H * 2));
  } else {
    is.ra = dn_rsrc4(w + (size_t)d.ex * H * I, (uint32_t)((size_t)H * I * 2));
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int R = 32 * wave + 16 * j + r;  // row of the tile
    int mrow;                              // row of the expert's matrix
    if (UP) {
      const int half = R >> 7, Rp = R & 127;
      const int col = d.g * DN_UP_COLS + half * 64 + (Rp & 63);
      mrow = Rp < 64 ? col : I + col;
    } else {
      mrow = d.g * DN_ROWS + R;
    }
    is.va[j] = (uint32_t)(mrow * K + q * 8) * 2;
    uint32_t vb = kDnPad;
    if (R < d.cnt) {
      if (UP) {  // an expanded index outside [0, T k) gathers a zero row
        const int e = perm[d.beg + R];
        if (e >= 0 && e < nmax) vb = (uint32_t)((e / k) * K + q * 8) * 2;
      } else {
        vb = (uint32_t)((d.beg + R) * K + q * 8) * 2;
      }
    }
    is.vb[j] = vb;
  }
}

// The fragment slot of this lane in a 1 KB block (row lane % 16, piece
// lane / 16), in u16x8 units.
__device__ __forceinline__ int dn_frag_slot(int lane) {
  const int r = lane & 15;
  return r * 4 + ((lane >> 4) ^ dn_swz(r));
}

// The 16 token groups of a pass are dealt to the four wave quarters
// strided (quarter w takes groups w, w + 4, w + 8, w + 12), so that the two
// waves of each SIMD share the work of a partly filled pass evenly; this is
// how many of its groups quarter wc multiplies for a pass of cnt entries
// (wave-uniform; the valid groups are the first ones).
__device__ __forceinline__ int dn_groups(int cnt, int wc) {
  const int ng = (cnt + 15) >> 4;
  return __builtin_amdgcn_readfirstlane(min(4, max(0, (ng - wc + 3) >> 2)));
}

// The LDS stage slots: S slots of 2 (up) or 3 (down) operand regions of
// 16 KB: the weight tile, the token rows and, for the down projection, the
// lo half of the intermediate.
constexpr int DN_REGION = DN_ROWS * 4;  // u16x8 per operand region

// A wave's fragments of one sub-stage: 8 weight fragments and 4 token
// fragments.
struct DnFrags {
  bf16x8 a[8], b[4];
};

__device__ __forceinline__ void dn_read(DnFrags& f, const u16x8* wa, const u16x8* wb) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.a[i] = __builtin_bit_cast(bf16x8, wa[i * 64]);
#pragma unroll
  for (int t = 0; t < 4; ++t) f.b[t] = __builtin_bit_cast(bf16x8, wb[t * 4 * 64]);
}

// The up projection's body. A stage is one 32-wide K slice of the weight and
// token tiles. Iteration c multiplies the fragments of stage c, read during
// iteration c - 1, while it reads those of stage c + 1 into the other
// register set; before that it makes stage c + 1 visible (the wave's own
// loads of it waited for, then the block barrier) and issues the loads of
// stage c + S - 1 into the slot stage c - 1 used, whose fragments every wave
// has multiplied by then. Stages run on across the block's tiles.
template <int S>
__device__ __forceinline__ void dn_body_up(const uint16_t* __restrict__ x,
                                           const int* __restrict__ perm, int k, int H, int I,
                                           int nmax, const uint16_t* __restrict__ w,
                                           const int* __restrict__ plan, int pmax,
                                           uint16_t* __restrict__ h_hi,
                                           uint16_t* __restrict__ h_lo, int NB, u16x8* lds) {
  constexpr int NI = 4;  // load instructions per wave and stage
  constexpr int SLOT = 2 * DN_REGION;
  if (plan[1] != 1) return;  // the staged kernels take this plan
  const int C = H / DN_K;
  const int G = I / DN_UP_COLS;
  const int P = plan[0];
  const int TT = P * G;
  const int b = xcd_block(blockIdx.x, NB);
  if (b >= TT) return;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wr = wave & 1, wc = wave >> 1;  // 128-row half, token quarter
  const u32x4 rb0 = dn_rsrc4(x, (uint32_t)((size_t)(nmax / k) * H * 2));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  // this lane's fragment slots: weight rows of its half, tokens of its quarter
  const int fs = dn_frag_slot(lane);
  const u16x8* const fa = lds + (wr * 8) * 64 + fs;
  const u16x8* const fb = lds + DN_REGION + wc * 64 + fs;

  // issue side: stage `issued` is the next to load
  DnIssue is;
  is.t = b;
  is.kc = 0;
  dn_issue_tile<true>(is, dn_tile(plan, pmax, b, G), perm, w, k, H, I, nmax, wave, lane);
  bool more = true;
  int issued = 0;
  auto issue = [&]() {
    if (!more) return;
    const uint32_t so = (uint32_t)is.kc * DN_K * 2;
    const uint32_t base = lds0 + (uint32_t)((issued % S) * SLOT) * 16u + (2 * wave) * 1024u;
    dn_dma(is.ra, base, is.va[0], so);
    dn_dma(is.ra, base + 1024u, is.va[1], so);
    dn_dma(rb0, base + DN_REGION * 16u, is.vb[0], so);
    dn_dma(rb0, base + DN_REGION * 16u + 1024u, is.vb[1], so);
    ++issued;
    if (++is.kc == C) {
      is.kc = 0;
      is.t += NB;
      if (is.t < TT)
        dn_issue_tile<true>(is, dn_tile(plan, pmax, is.t, G), perm, w, k, H, I, nmax, wave, lane);
      else
        more = false;
    }
  };
  // Wait until this wave's loads of stage `st` have landed, then meet the
  // block: stage st is visible to every wave.
  auto publish = [&](int st) {
    const int after = issued - st - 1;  // stages issued after st
    if (after >= 2) __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * NI));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(0x0f70 | NI);
    else __builtin_amdgcn_s_waitcnt(0x0f70);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto read = [&](DnFrags& f, int st) {
    const int sl = (st % S) * SLOT;
    dn_read(f, fa + sl, fb + sl);
  };

  for (int i = 0; i + 1 < S; ++i) issue();
  publish(0);

  DnTile cur = dn_tile(plan, pmax, b, G);
  int kc = 0;  // stage of the current tile
  int c = 0;   // stage of the block
  int nv = dn_groups(cur.cnt, wc);
  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // SwiGLU of the finished tile: gate group f pairs with up group f + 4.
  auto epilogue = [&]() {
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = (t * 4 + wc) * 16 + (lane & 15);
      if (n < cur.cnt) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          u16x4 hi, lo;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gg = acc[f * 4 + t][j], uu = acc[(f + 4) * 4 + t][j];
            const float av = gg / (1.0f + expf(-gg)) * uu;
            hi[j] = f32_to_bf16_bits(av);
            lo[j] = f32_to_bf16_bits(av - bf16_bits_to_f32(hi[j]));
          }
          const int col = cur.g * DN_UP_COLS + wr * 64 + f * 16 + (lane >> 4) * 4;
          const size_t o = (size_t)(cur.beg + n) * I + col;
          *reinterpret_cast<u16x4*>(h_hi + o) = hi;
          *reinterpret_cast<u16x4*>(h_lo + o) = lo;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  auto mma = [&](const DnFrags& f) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t >= nv) break;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        acc[r * 4 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[r], f.b[t], acc[r * 4 + t], 0, 0, 0);
    }
  };

  // Multiply stage c from `cf` while reading stage c + 1 into `nf`. Returns
  // false after the block's last stage.
  auto iter = [&](const DnFrags& cf, DnFrags& nf) -> bool {
    const bool last = c + 1 == issued && !more;  // no stage after c
    if (!last) {
      publish(c + 1);
      issue();
    }
    // (after the block's last stage a dummy read of stage c, so that the
    // reads never sit in a branch: the compiler then waits only for the
    // previous iteration's reads before the MFMAs, not for these)
    read(nf, last ? c : c + 1);
    mma(cf);
    ++c;
    if (++kc == C) {
      epilogue();
      kc = 0;
      const int nt = cur.t + NB;
      if (nt >= TT) return false;
      cur = dn_tile(plan, pmax, nt, G);
      nv = dn_groups(cur.cnt, wc);
    }
    return true;
  };

  DnFrags f0, f1;
  read(f0, 0);
  if (iter(f0, f1)) {
    while (iter(f1, f0) && iter(f0, f1)) {
    }
  }
}

// The down projection's fragments of one stage for one wave, read from LDS
// in one asm block that also waits for them: the weight fragments (8 blocks
// of 1 KB from byte address `a`), the hi fragments (every fourth 1 KB block
// from `b`: the wave quarter's token groups) and the lo fragments (likewise
// from `c`), each lane at its fragment slot. The
// loads that fill a stage are published to the block by the stage's explicit
// wait and barrier. The outputs are early-clobber: the asm's later reads
// still use the address registers, which no output may share.
__device__ __forceinline__ void dn_frags(bf16x8 (&af)[8], bf16x8 (&bf)[4], bf16x8 (&cf)[4],
                                         uint32_t a, uint32_t b, uint32_t c) {
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %16 offset:1024\n"
      "ds_read_b128 %2, %16 offset:2048\n"
      "ds_read_b128 %3, %16 offset:3072\n"
      "ds_read_b128 %4, %16 offset:4096\n"
      "ds_read_b128 %5, %16 offset:5120\n"
      "ds_read_b128 %6, %16 offset:6144\n"
      "ds_read_b128 %7, %16 offset:7168\n"
      "ds_read_b128 %8, %17\n"
      "ds_read_b128 %9, %17 offset:4096\n"
      "ds_read_b128 %10, %17 offset:8192\n"
      "ds_read_b128 %11, %17 offset:12288\n"
      "ds_read_b128 %12, %18\n"
      "ds_read_b128 %13, %18 offset:4096\n"
      "ds_read_b128 %14, %18 offset:8192\n"
      "ds_read_b128 %15, %18 offset:12288\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]), "=&v"(af[5]),
        "=&v"(af[6]), "=&v"(af[7]), "=&v"(bf[0]), "=&v"(bf[1]), "=&v"(bf[2]), "=&v"(bf[3]),
        "=&v"(cf[0]), "=&v"(cf[1]), "=&v"(cf[2]), "=&v"(cf[3])
      : "v"(a), "v"(b), "v"(c)
      : "memory");
}

// The down projection's body: one sub-stage per stage, every fragment of the
// stage (weights, hi, lo) read at its start, the MFMAs after. At stage i a
// wave waits for its own loads of stage i, meets the block (every wave's
// loads of stage i have landed and every wave has finished stage i - 1),
// issues the loads of stage i + S - 1 into the slot stage i - 1 used, and
// multiplies stage i: two stages of loads in flight behind the one
// multiplied. (The up projection's read-ahead of the next stage's fragments
// needs a second register set, which the hi + lo fragments leave no room
// for; with the hi and lo halves as separate sub-stages and one stage of
// loads in flight the down projection measured 3.14 against 2.92 ms at the
// probe shape.)
template <int S>
__device__ __forceinline__ void dn_body_down(const uint16_t* __restrict__ h_hi,
                                             const uint16_t* __restrict__ h_lo, int k, int H,
                                             int I, int nmax, const uint16_t* __restrict__ w,
                                             const int* __restrict__ plan, int pmax,
                                             float* __restrict__ out, int NB, u16x8* lds) {
  constexpr int NI = 6;  // load instructions per wave and stage
  constexpr int SLOT = 3 * DN_REGION;
  if (plan[1] != 1) return;  // the staged kernels take this plan
  const int C = I / DN_K;
  const int G = H / DN_ROWS;
  const int P = plan[0];
  const int TT = P * G;
  const int b = xcd_block(blockIdx.x, NB);
  if (b >= TT) return;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wr = wave & 1, wc = wave >> 1;
  const u32x4 rb0 = dn_rsrc4(h_hi, (uint32_t)((size_t)nmax * I * 2));
  const u32x4 rb1 = dn_rsrc4(h_lo, (uint32_t)((size_t)nmax * I * 2));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  const uint32_t fs = (uint32_t)dn_frag_slot(lane) * 16u;
  const uint32_t fa = lds0 + (uint32_t)(wr * 8) * 1024u + fs;
  const uint32_t fb = lds0 + DN_REGION * 16u + (uint32_t)wc * 1024u + fs;

  DnIssue is;
  is.t = b;
  is.kc = 0;
  dn_issue_tile<false>(is, dn_tile(plan, pmax, b, G), nullptr, w, k, H, I, nmax, wave, lane);
  bool more = true;
  int issued = 0;
  auto issue = [&]() {
    if (!more) return;
    const uint32_t so = (uint32_t)is.kc * DN_K * 2;
    const uint32_t base = lds0 + (uint32_t)((issued % S) * SLOT) * 16u + (2 * wave) * 1024u;
    dn_dma(is.ra, base, is.va[0], so);
    dn_dma(is.ra, base + 1024u, is.va[1], so);
    dn_dma(rb0, base + DN_REGION * 16u, is.vb[0], so);
    dn_dma(rb0, base + DN_REGION * 16u + 1024u, is.vb[1], so);
    dn_dma(rb1, base + 2 * DN_REGION * 16u, is.vb[0], so);
    dn_dma(rb1, base + 2 * DN_REGION * 16u + 1024u, is.vb[1], so);
    ++issued;
    if (++is.kc == C) {
      is.kc = 0;
      is.t += NB;
      if (is.t < TT)
        dn_issue_tile<false>(is, dn_tile(plan, pmax, is.t, G), nullptr, w, k, H, I, nmax, wave,
                             lane);
      else
        more = false;
    }
  };
  for (int i = 0; i + 1 < S; ++i) issue();

  DnTile cur = dn_tile(plan, pmax, b, G);
  int kc = 0, done = 0;
  int nv = dn_groups(cur.cnt, wc);
  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (;;) {
    const int after = issued - done - 1;  // stages issued after this one
    if (after >= 2) __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * NI));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(0x0f70 | NI);
    else __builtin_amdgcn_s_waitcnt(0x0f70);
    __builtin_amdgcn_s_barrier();
    issue();
    if (nv > 0) {
      const uint32_t sl = (uint32_t)((done % S) * SLOT) * 16u;
      bf16x8 af[8], bh[4], bl[4];
      dn_frags(af, bh, bl, fa + sl, fb + sl, fb + sl + DN_REGION * 16u);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t >= nv) break;
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          acc[f * 4 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[f], bh[t], acc[f * 4 + t], 0, 0, 0);
          acc[f * 4 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[f], bl[t], acc[f * 4 + t], 0, 0, 0);
        }
      }
    }
    ++done;
    if (++kc == C) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = (t * 4 + wc) * 16 + (lane & 15);
        if (n < cur.cnt) {
#pragma unroll
          for (int f = 0; f < 8; ++f) {
            const int row = cur.g * DN_ROWS + wr * 128 + f * 16 + (lane >> 4) * 4;
            *reinterpret_cast<f32x4*>(out + (size_t)(cur.beg + n) * H + row) = acc[f * 4 + t];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      kc = 0;
      const int nt = cur.t + NB;
      if (nt >= TT) return;
      cur = dn_tile(plan, pmax, nt, G);
      nv = dn_groups(cur.cnt, wc);
    }
  }
}

__global__ __launch_bounds__(DN_THREADS, 1) void ffn_dense_up_kernel(
    const uint16_t* __restrict__ x, const int* __restrict__ perm, int k, int H, int I, int nmax,
    const uint16_t* __restrict__ w1, const int* __restrict__ plan, int pmax,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo, int NB) {
  __shared__ u16x8 lds[DN_UP_STAGES * 2 * DN_REGION];
  dn_body_up<DN_UP_STAGES>(x, perm, k, H, I, nmax, w1, plan, pmax, h_hi, h_lo, NB, lds);
}

__global__ __launch_bounds__(DN_THREADS, 1) void ffn_dense_down_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int k, int H, int I,
    int nmax, const uint16_t* __restrict__ w2, const int* __restrict__ plan, int pmax,
    float* __restrict__ out, int NB) {
  __shared__ u16x8 lds[DN_DOWN_STAGES * 3 * DN_REGION];
  dn_body_down<DN_DOWN_STAGES>(h_hi, h_lo, k, H, I, nmax, w2, plan, pmax, out, NB, lds);
}

}  // namespace

// Resident blocks of the dense kernels on the current device (one per CU:
// each holds 128 or 144 KB of LDS).
int ffn_dense_blocks() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0, a = 0, b = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, ffn_dense_up_kernel, DN_THREADS, 0) !=
            hipSuccess || a <= 0)
      a = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, ffn_dense_down_kernel, DN_THREADS, 0) !=
            hipSuccess || b <= 0)
      b = 1;
    cached[dev] = std::min(a, b) * cus;
  }
  return cached[dev];
}

// Shapes the dense kernels take: 128-column up tiles, 256-row down tiles,
// 32-wide K stages, and 32-bit buffer offsets for the token rows, the
// intermediate and one expert's weights.
bool ffn_dense_shape_ok(int T, int k, int H, int I) {
  const size_t lim = (size_t)1 << 31;
  return H % DN_ROWS == 0 && I % DN_UP_COLS == 0 && H % DN_K == 0 && I % DN_K == 0 &&
         (size_t)T * H * 2 < lim && (size_t)T * k * I * 2 < lim && (size_t)2 * I * H * 2 < lim;
}

int ffn_dense_pass_tokens() { return DN_TOK; }

// The up and down kernels over the pass plan `plan` (passes of at most 256
// entries, written beforehand); they return at once unless the plan names
// the dense kernels.
hipError_t launch_ffn_dense_up(const uint16_t* x, const int* perm, int k, int H, int I, int nmax,
                               const uint16_t* w1, const int* plan, int pmax, uint16_t* h_hi,
                               uint16_t* h_lo, hipStream_t stream) {
  const int nb = ffn_dense_blocks();
  hipLaunchKernelGGL(ffn_dense_up_kernel, dim3(nb), dim3(DN_THREADS), 0, stream, x, perm, k, H, I,
                     nmax, w1, plan, pmax, h_hi, h_lo, nb);
  return hipGetLastError();
}

hipError_t launch_ffn_dense_down(const uint16_t* h_hi, const uint16_t* h_lo, int k, int H, int I,
                                 int nmax, const uint16_t* w2, const int* plan, int pmax,
                                 float* out, hipStream_t stream) {
  const int nb = ffn_dense_blocks();
  hipLaunchKernelGGL(ffn_dense_down_kernel, dim3(nb), dim3(DN_THREADS), 0, stream, h_hi, h_lo, k,
                     H, I, nmax, w2, plan, pmax, out, nb);
  return hipGetLastError();
}

}  // namespace moe
