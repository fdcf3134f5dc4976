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
// 64 tokens each (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//
// Staging: each 32-wide K stage of both operands goes HBM/L2 -> LDS by
// buffer loads that write LDS directly (one 1 KB block of 16 rows x 64 bytes
// per wave instruction, no VGPR round trip), several stages ahead (4 LDS
// stages for the up projection, 3 for the down projection, whose token
// operand is the hi and lo halves of the intermediate). Rows past a pass's
// entries carry a buffer offset beyond the resource, which reads zeros with
// no memory request. Within a block, 16-byte piece q of row r sits at slot
// q ^ ((r >> 1) & 3): the MFMA fragment reads (16 rows, one piece each, per
// 16 lanes) then run without bank conflicts. Measured on MI355X with a probe
// of such reads (16 waves per CU): 490 B/ns per CU conflict-free, against
// 280 B/ns and 4 conflict cycles per read for rows without the XOR, for
// rows padded to 144 bytes, for q ^ (r & 3) and for q ^ (((r >> 1) ^
// (r >> 3)) & 3).
//
// Pipeline: one block barrier per stage. At stage i a wave waits for its own
// loads of stage i (vmcnt), meets the block (so every wave's loads of stage i
// have landed and every wave has finished stage i - 1), issues the loads of
// stage i + S - 1 into the buffer stage i - 1 used, and multiplies stage i.
// Stages run on across tiles (a block's next tile starts loading while the
// current one finishes), and a tile's epilogue writes its outputs right after
// its last stage.
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

// One operand of one stage: 256 rows x 32 bf16 (16 blocks of 16 rows x 64 B).
typedef u16x8 dn_buf_t[DN_ROWS * 4];
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ int dn_swz(int r) { return (r >> 1) & 3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dn_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// One 1 KB block (16 rows) of a stage, loaded by the whole wave straight into
// LDS at dst: lane i fills slot i (row i / 4, slot i % 4).
__device__ __forceinline__ void dn_dma(__amdgpu_buffer_rsrc_t rs, u16x8* dst, uint32_t voff,
                                       uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 16, voff, soff, 0, 0);
}

// Plan entries of a tile (pass-major numbering t = pass * G + g).
struct DnTile {
  int t, ex, beg, cnt, g;
};

__device__ __forceinline__ DnTile dn_tile(const int* __restrict__ plan, int pmax, int t, int G) {
  const int pass = t / G;
  DnTile d;
  d.t = t;
  d.g = t - pass * G;
  d.ex = plan[4 + pass];
  d.beg = plan[4 + pmax + pass];
  d.cnt = plan[4 + 2 * pmax + pass];
  return d;
}

// The loads a wave issues for one stage: blocks 2w and 2w + 1 of the weight
// tile and of the token tile (and of the lo half for the down projection).
struct DnIssue {
  __amdgpu_buffer_rsrc_t ra;  // the tile's expert matrix
  uint32_t va[2], vb[2];      // this lane's byte offsets in its two blocks
  int t, kc;                  // tile and stage being issued
};

template <bool UP>
__device__ __forceinline__ void dn_issue_tile(DnIssue& is, const DnTile& d,
                                              const int* __restrict__ perm, const uint16_t* w,
                                              int k, int H, int I, int nmax, int wave, int lane) {
  const int K = UP ? H : I;
  const int r = lane >> 2, q = (lane & 3) ^ dn_swz(r);
  if (UP) {
    is.ra = dn_rsrc(w + (size_t)d.ex * 2 * I * H, (uint32_t)((size_t)2 * I * H * 2));
  } else {
    is.ra = dn_rsrc(w + (size_t)d.ex * H * I, (uint32_t)((size_t)H * I * 2));
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

// LDS stage slot PH: the weight tile at +0, the token rows at +1024 and, for
// the down projection, the lo half at +2048 (u16x8 units). Each slot is its
// own LDS array, so the compiler can tell a stage's LDS reads from the loads
// in flight into the other slots and waits only for the loads of the slot it
// reads (with one array per operand and slot, more arrays than it tracks).
template <bool UP, int PH>
__device__ __forceinline__ u16x8* dn_slot() {
  __shared__ u16x8 buf[(UP ? 2 : 3) * DN_ROWS * 4];
  return buf;
}

// The kernel body; S stage slots.
// A stage's operand fragments of one wave, read from LDS in one asm block
// that also waits for them: the weight fragments (8 blocks of 1 KB from
// `a`), the token fragments (4 blocks from `b`) and, for the down
// projection, the lo half (4 blocks from `c`; NC = 4), each lane at its
// fragment slot. The loads that fill a stage are published to the block by
// the stage's explicit wait and barrier; reading through asm keeps the
// compiler from adding waits of its own for the loads in flight into the
// other stage slots, which it cannot tell apart across the loop.
template <int NC>
__device__ __forceinline__ void dn_frags(bf16x8 (&af)[8], bf16x8 (&bf)[4], bf16x8 (&cf)[4],
                                         uint32_t a, uint32_t b, uint32_t c) {
  if constexpr (NC == 0) {
    asm volatile(
        "ds_read_b128 %0, %12\n"
        "ds_read_b128 %1, %12 offset:1024\n"
        "ds_read_b128 %2, %12 offset:2048\n"
        "ds_read_b128 %3, %12 offset:3072\n"
        "ds_read_b128 %4, %12 offset:4096\n"
        "ds_read_b128 %5, %12 offset:5120\n"
        "ds_read_b128 %6, %12 offset:6144\n"
        "ds_read_b128 %7, %12 offset:7168\n"
        "ds_read_b128 %8, %13\n"
        "ds_read_b128 %9, %13 offset:1024\n"
        "ds_read_b128 %10, %13 offset:2048\n"
        "ds_read_b128 %11, %13 offset:3072\n"
        "s_waitcnt lgkmcnt(0)\n"
        : "=v"(af[0]), "=v"(af[1]), "=v"(af[2]), "=v"(af[3]), "=v"(af[4]), "=v"(af[5]),
          "=v"(af[6]), "=v"(af[7]), "=v"(bf[0]), "=v"(bf[1]), "=v"(bf[2]), "=v"(bf[3])
        : "v"(a), "v"(b)
        : "memory");
    (void)c;
    (void)cf;
  } else {
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
        "ds_read_b128 %9, %17 offset:1024\n"
        "ds_read_b128 %10, %17 offset:2048\n"
        "ds_read_b128 %11, %17 offset:3072\n"
        "ds_read_b128 %12, %18\n"
        "ds_read_b128 %13, %18 offset:1024\n"
        "ds_read_b128 %14, %18 offset:2048\n"
        "ds_read_b128 %15, %18 offset:3072\n"
        "s_waitcnt lgkmcnt(0)\n"
        : "=v"(af[0]), "=v"(af[1]), "=v"(af[2]), "=v"(af[3]), "=v"(af[4]), "=v"(af[5]),
          "=v"(af[6]), "=v"(af[7]), "=v"(bf[0]), "=v"(bf[1]), "=v"(bf[2]), "=v"(bf[3]),
          "=v"(cf[0]), "=v"(cf[1]), "=v"(cf[2]), "=v"(cf[3])
        : "v"(a), "v"(b), "v"(c)
        : "memory");
  }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <bool UP, int S>
__device__ __forceinline__ void dn_body(const uint16_t* __restrict__ b0src,
                                        const uint16_t* __restrict__ b1src,
                                        const int* __restrict__ perm, int k, int H, int I,
                                        int nmax, const uint16_t* __restrict__ w,
                                        const int* __restrict__ plan, int pmax,
                                        uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo,
                                        float* __restrict__ out, int NB) {
  constexpr int NI = UP ? 4 : 6;  // load instructions per wave and stage
  const int K = UP ? H : I;
  const int C = K / DN_K;
  const int G = UP ? I / DN_UP_COLS : H / DN_ROWS;
  if (plan[1] != 1) return;  // the staged kernels take this plan
  const int P = plan[0];
  const int TT = P * G;
  const int b = xcd_block(blockIdx.x, NB);
  if (b >= TT) return;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wr = wave & 1, wc = wave >> 1;  // 128-row half, 64-token quarter
  const __amdgpu_buffer_rsrc_t rb0 =
      dn_rsrc(b0src, (uint32_t)(UP ? (size_t)(nmax / k) * H * 2 : (size_t)nmax * I * 2));
  const __amdgpu_buffer_rsrc_t rb1 = dn_rsrc(b1src, (uint32_t)((size_t)nmax * I * 2));
  const int fs = dn_frag_slot(lane);

  // issue side: runs S - 1 stages ahead of the compute side
  DnIssue is;
  is.t = b;
  is.kc = 0;
  dn_issue_tile<UP>(is, dn_tile(plan, pmax, b, G), perm, w, k, H, I, nmax, wave, lane);
  bool more = true;  // stages left to issue
  int issued = 0;    // stages issued so far
  auto issue = [&](u16x8* slot) {
    if (!more) return;
    u16x8* const na = slot;
    u16x8* const nb_ = slot + DN_ROWS * 4;
    u16x8* const nc = slot + 2 * DN_ROWS * 4;
    const uint32_t so = (uint32_t)is.kc * DN_K * 2;
    dn_dma(is.ra, na + (2 * wave) * 64, is.va[0], so);
    dn_dma(is.ra, na + (2 * wave + 1) * 64, is.va[1], so);
    dn_dma(rb0, nb_ + (2 * wave) * 64, is.vb[0], so);
    dn_dma(rb0, nb_ + (2 * wave + 1) * 64, is.vb[1], so);
    if (!UP) {
      dn_dma(rb1, nc + (2 * wave) * 64, is.vb[0], so);
      dn_dma(rb1, nc + (2 * wave + 1) * 64, is.vb[1], so);
    }
    ++issued;
    if (++is.kc == C) {
      is.kc = 0;
      is.t += NB;
      if (is.t < TT)
        dn_issue_tile<UP>(is, dn_tile(plan, pmax, is.t, G), perm, w, k, H, I, nmax, wave, lane);
      else
        more = false;
    }
  };
  issue(dn_slot<UP, 0>());
  issue(dn_slot<UP, 1>());
  if constexpr (S == 4) issue(dn_slot<UP, 2>());

  // compute side
  DnTile cur = dn_tile(plan, pmax, b, G);
  int kc = 0;
  int nv = __builtin_amdgcn_readfirstlane(min(4, max(0, (cur.cnt - wc * 64 + 15) >> 4)));
  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto epilogue = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = wc * 64 + t * 16 + (lane & 15);
      if (n < cur.cnt) {
        if (UP) {
          typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
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
        } else {
#pragma unroll
          for (int f = 0; f < 8; ++f) {
            const int row = cur.g * DN_ROWS + wr * 128 + f * 16 + (lane >> 4) * 4;
            *reinterpret_cast<f32x4*>(out + (size_t)(cur.beg + n) * H + row) = acc[f * 4 + t];
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // Multiply one stage held in a slot: every fragment is read first, then
  // the MFMAs of the token groups that hold entries.
  auto mma = [&](const u16x8* slot) {
    if (nv == 0) return;
    bf16x8 af[8], bh[4], bl[4];
    const u16x8* const sa = slot + (wr * 8) * 64 + fs;
    const u16x8* const sb = slot + DN_ROWS * 4 + (wc * 4) * 64 + fs;
    dn_frags<UP ? 0 : 4>(af, bh, bl, lds_addr(sa), lds_addr(sb),
                         lds_addr(sb + DN_ROWS * 4));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t >= nv) break;
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        acc[f * 4 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[f], bh[t], acc[f * 4 + t], 0, 0, 0);
        if (!UP)
          acc[f * 4 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[f], bl[t], acc[f * 4 + t], 0, 0, 0);
      }
    }
  };

  int done = 0;  // stages computed
  // Stage `done` sits in slot PH = done % S: wait for this wave's loads of
  // it, meet the block, issue stage done + S - 1 into slot (PH + S - 1) % S
  // (the one stage done - 1 used), multiply slot PH, and end the tile after
  // its last stage. Returns false after the block's last stage.
  auto step = [&](auto ph) -> bool {
    constexpr int PH = decltype(ph)::value;
    constexpr int NX = (PH + S - 1) % S;
    const int ahead = issued - done - 1;  // stages issued after this one
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * NI));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0f70 | NI);
    else __builtin_amdgcn_s_waitcnt(0x0f70);
    __builtin_amdgcn_s_barrier();
    issue(dn_slot<UP, NX>());
    mma(dn_slot<UP, PH>());
    ++done;
    if (++kc == C) {
      epilogue();
      kc = 0;
      const int nt = cur.t + NB;
      if (nt >= TT) return false;
      cur = dn_tile(plan, pmax, nt, G);
      nv = __builtin_amdgcn_readfirstlane(min(4, max(0, (cur.cnt - wc * 64 + 15) >> 4)));
    }
    return true;
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  if constexpr (S == 4) {
    while (step(P0{}) && step(P1{}) && step(P2{}) && step(P3{})) {
    }
  } else {
    while (step(P0{}) && step(P1{}) && step(P2{})) {
    }
  }
}

__global__ __launch_bounds__(DN_THREADS, 1) void ffn_dense_up_kernel(
    const uint16_t* __restrict__ x, const int* __restrict__ perm, int k, int H, int I, int nmax,
    const uint16_t* __restrict__ w1, const int* __restrict__ plan, int pmax,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo, int NB) {
  dn_body<true, DN_UP_STAGES>(x, x, perm, k, H, I, nmax, w1, plan, pmax, h_hi, h_lo, nullptr, NB);
}

__global__ __launch_bounds__(DN_THREADS, 1) void ffn_dense_down_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int k, int H, int I,
    int nmax, const uint16_t* __restrict__ w2, const int* __restrict__ plan, int pmax,
    float* __restrict__ out, int NB) {
  dn_body<false, DN_DOWN_STAGES>(h_hi, h_lo, nullptr, k, H, I, nmax, w2, plan, pmax, nullptr,
                                 nullptr, out, NB);
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
