// The pass plan of the persistent grouped-FFN kernels (ffn_sk.hip): the list
// of passes (local expert, first entry, entries) that the kernels deal out as
// tiles, and the zeroed arrival counters of their cross-block fixup. Written
// either by ffn_plan_kernel or, in the layer (moe_forward), by the routing's
// permutation kernel right after it has the offsets, which saves a launch.
#pragma once

#include "device.h"

namespace moe {

// Plan layout (ints): [0] passes P, [1] kernel family (0: the staged or
// K-split kernels, 1: the dense kernels), then pass_expert[pmax],
// pass_beg[pmax], pass_cnt[pmax], and per pass its expert's first pass
// pass_first[pmax] and number of passes pass_num[pmax].
constexpr int kPlanArrays = 5;
struct PlanView {
  int* hdr;
  int* expert;
  int* beg;
  int* cnt;
  int* first;
  int* num;
};

__device__ __forceinline__ PlanView plan_view(int* plan, int pmax) {
  return PlanView{plan, plan + 4, plan + 4 + pmax, plan + 4 + 2 * pmax, plan + 4 + 3 * pmax,
                  plan + 4 + 4 * pmax};
}

// Where a plan goes: `plan` (NULL: no plan to write), passes of at most nr
// entries over entries [0, nmax), and `ncounters` counters to zero. With
// nr_dense > 0 the writer picks the dense kernels, with passes of nr_dense
// entries, when the local entries reach dense_min per local expert: only the
// device knows the entry counts, and on an expert share they can be a small
// fraction of the T k selections.
struct PlanOut {
  int* plan;
  int pmax, nr, nmax;
  int* counters;
  int ncounters;
  int nr_dense, dense_min;
};

// The plan from the exclusive scan `off` of the local experts' entry counts
// (LDS, off[L] = entries in all). One block of nt threads (blockDim.x), every
// thread calls it; `s_pass` is LDS scratch of L + 1 + 16 ints. The callers
// zero the counters.
__device__ inline void write_ffn_plan(const int* off, int L, const PlanOut& po, int* s_pass,
                                      int nt) {
  const int tid = threadIdx.x;
  const int n_local = max(0, min(off[L], po.nmax)) - max(0, min(off[0], po.nmax));
  const bool dense = po.nr_dense > 0 && (long)n_local >= (long)po.dense_min * L;
  const int nr = dense ? po.nr_dense : po.nr;
  for (int i = tid; i < L; i += nt) {
    const int b = max(0, min(off[i], po.nmax));
    const int e = max(b, min(off[i + 1], po.nmax));
    s_pass[i] = (e - b + nr - 1) / nr;
  }
  __syncthreads();
  block_exclusive_scan(s_pass, L, s_pass + L + 1, nt);
  const PlanView pv = plan_view(po.plan, po.pmax);
  for (int i = tid; i < L; i += nt) {
    const int b = max(0, min(off[i], po.nmax));
    const int e = max(b, min(off[i + 1], po.nmax));
    const int q0 = s_pass[i], np = s_pass[i + 1] - q0;
    for (int q = q0, t = b; t < e; ++q, t += nr) {
      pv.expert[q] = i;
      pv.beg[q] = t;
      pv.cnt[q] = min(nr, e - t);
      pv.first[q] = q0;
      pv.num[q] = np;
    }
  }
  if (tid == 0) {
    pv.hdr[0] = s_pass[L];
    pv.hdr[1] = dense ? 1 : 0;
  }
}

}  // namespace moe
