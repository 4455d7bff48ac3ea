// The two-group ("ping-pong") phase schedule of the fused attention kernels,
// shared by the INT8/FP8 and the FP4 kernels.
//
// One work-group = 8 waves = two groups of four, each group one 128-query tile
// of the same (batch, head). The groups share the K/V tiles in LDS (double
// buffered) and run half a tile apart: while one group is in its matrix phase
// X(t) = PV(t-1) + QK^T(t), the other is in its vector phase Y(t) (softmax of
// its current tile), so on every SIMD one wave keeps the matrix cores busy
// while the other issues vector instructions. Every phase ends at a
// work-group barrier.
//
// Global phase p: group 0 runs X(t) at p = 2t and Y(t) at p = 2t + 1; group 1
// one phase later. K(t) is read in phases 2t and 2t+1, V(t-1) in the same two
// phases. Group 0 issues the load of K(t+1) in phase 2t (into the buffer
// K(t-1) left), group 1 the load of V(t) in phase 2t+1 (into the buffer V(t-2)
// left), each during its matrix phase; both land by the end of phase 2t+1.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace sage {

// Pins a value in registers at this point: it must be computed before here and
// cannot be sunk past it. Used to keep each phase's work inside its phase (the
// barriers order memory only). Emits no instruction.
template <typename V>
__device__ __forceinline__ void pin(V& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_loads_barrier() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// The two groups' phase sequence for one work-group (the order described
// above), shared by the kernels that run this schedule. n: tiles this group
// attends to (0 for a group past the queries); n_wg: the work-group's (the
// longer group's) tile count. The phase functions:
//   x_phase(par, t, do_pv, do_qk)   X(t) with buffer parity par (compile time)
//   x_phase_loading(par, t)         X(t) of a steady pair, issuing this
//                                   group's loads between its products
//   x_phase_rt(t, do_pv, do_qk)     X(t), parity known at run time
//   y_phase(t, masked)              Y(t); masked: std::true_type on the tile
//                                   that may need masking (a group's last)
//   loads_k(par, t) / loads_v(par, t) and their run-time-parity forms: group
//   0 issues K(t+1), group 1 V(t).
// The two barriers: the one between the phases of a pair, and the one that
// ends a pair after waiting for this wave's loads. (A phase-trace build passes
// timing wrappers.)
struct PhaseBarrier {
  __device__ __forceinline__ void operator()() const { barrier_only(); }
};
struct PairBarrier {
  __device__ __forceinline__ void operator()() const { wait_loads_barrier(); }
};

template <class XP, class XL, class XR, class YP, class LK, class LV, class LKR, class LVR,
          class BA = PhaseBarrier, class BW = PairBarrier>
__device__ __forceinline__ void run_pingpong(int grp, int n, int n_wg, const XP& x_phase,
                                             const XL& x_phase_loading, const XR& x_phase_rt, const YP& y_phase,
                                             const LK& loads_k, const LV& loads_v, const LKR& loads_k_rt,
                                             const LVR& loads_v_rt, const BA& barrier_only = BA{},
                                             const BW& wait_loads_barrier = BW{}) {
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  using Masked = std::true_type;
  using Full = std::false_type;

  if (grp == 0) {
    // group 0, pair t: X(t) | Y(t); issues K(t+1) in X(t)
    if (n > 0) {
      x_phase(Even{}, 0, false, true);
      loads_k(Even{}, 0);
      barrier_only();
      if (n == 1) y_phase(0, Masked{}); else y_phase(0, Full{});
      wait_loads_barrier();
      auto steady = [&](auto par, int t) __attribute__((always_inline)) {
        x_phase_loading(par, t);
        barrier_only();
        y_phase(t, Full{});
        wait_loads_barrier();
      };
      int t = 1;
      for (; t + 1 <= n - 2; t += 2) {
        steady(Odd{}, t);
        steady(Even{}, t + 1);
      }
      if (t <= n - 2) { steady(Odd{}, t); ++t; }
      if (n >= 2) {
        loads_k_rt(n - 1);
        x_phase_rt(n - 1, true, true);
        barrier_only();
        y_phase(n - 1, Masked{});
        wait_loads_barrier();
      }
      loads_k_rt(n);
      x_phase_rt(n, true, false);
      barrier_only();
      wait_loads_barrier();
    }
    for (int t = n + (n > 0 ? 1 : 0); t <= n_wg; ++t) {
      loads_k_rt(t);
      barrier_only();
      wait_loads_barrier();
    }
  } else {
    // group 1, pair t: Y(t-1) | X(t); issues V(t) in X(t)
    if (n > 0) {
      barrier_only();
      x_phase(Even{}, 0, false, true);
      loads_v(Even{}, 0);
      wait_loads_barrier();
      auto steady = [&](auto par, int t) __attribute__((always_inline)) {
        y_phase(t - 1, Full{});
        barrier_only();
        x_phase_loading(par, t);
        wait_loads_barrier();
      };
      int t = 1;
      for (; t + 1 <= n - 1; t += 2) {
        steady(Odd{}, t);
        steady(Even{}, t + 1);
      }
      if (t <= n - 1) { steady(Odd{}, t); ++t; }
      // t == n (== n_wg): masked last tile's softmax, then PV(n - 1); no V(n)
      y_phase(n - 1, Masked{});
      barrier_only();
      x_phase_rt(n, true, false);
      wait_loads_barrier();
    }
    for (int t = n + (n > 0 ? 1 : 0); t <= n_wg; ++t) {
      barrier_only();
      loads_v_rt(t);
      wait_loads_barrier();
    }
  }
}

}  // namespace sage
