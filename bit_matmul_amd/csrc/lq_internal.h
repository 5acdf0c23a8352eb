// Internal declarations of liblq: device helpers shared by the kernels and the
// launchers that the C ABI (api.cpp) calls. Not installed, not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lq {

constexpr int kPanelRows = 16;     // rows per packed panel
constexpr int kTileCols = 512;     // lifted columns per full packed tile
constexpr int kTileBytes = 1024;   // 16 rows x 512 bits

// Geometry of a packed N x L sign matrix (see include/lq.h for the layout).
struct PackedGeom {
  int64_t N, L;
  int64_t panels;       // N / 16
  int64_t panel_bytes;  // 2 L
  int full_tiles;       // L / 512
  int tail_bytes;       // (L % 512) / 8 bytes per row in the tail
  int ext_tiles;        // full tiles plus one for a non-empty tail
};

inline PackedGeom make_geom(int64_t N, int64_t L) {
  PackedGeom g;
  g.N = N;
  g.L = L;
  g.panels = N / kPanelRows;
  g.panel_bytes = 2 * L;
  g.full_tiles = (int)(L / kTileCols);
  g.tail_bytes = (int)((L % kTileCols) / 8);
  g.ext_tiles = g.full_tiles + (g.tail_bytes ? 1 : 0);
  return g;
}

// bf16 bits of f, rounded to nearest, ties to even (gfx950's
// v_cvt_pk_bf16_f32; fp32 denormals are kept, so every finite value rounds
// as the IEEE rule says; NaNs come out quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(unsigned short, (__bf16)f);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// The 16-byte slot (g, r) of full tile q of one panel, as four 32-bit words:
// word u, bit b = sign bit of row r at tile column 128u + 32g + b. A
// non-temporal load: the products that use it read each weight byte once.
__device__ __forceinline__ uint4 load_full_slot(const uint8_t* __restrict__ panel, int q, int g,
                                                int r) {
  typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
  const v4u_t v = __builtin_nontemporal_load(
      reinterpret_cast<const v4u_t*>(panel + (int64_t)q * kTileBytes + 16 * (16 * g + r)));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same slot of the partial tail tile, assembled from the row-major tail
// bytes (columns beyond L read as 0, sign +1). Branch-free: every lane loads
// 16 bytes at clamped in-bounds offsets and masks the ones past the row.
__device__ __forceinline__ uint4 load_tail_slot(const uint8_t* __restrict__ panel, int full_tiles,
                                                int tail_bytes, int g, int r) {
  const uint8_t* row = panel + (int64_t)full_tiles * kTileBytes + r * tail_bytes;
  uint32_t w[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    uint32_t v = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = 16 * u + 4 * g + k;
      const uint32_t byte = row[t < tail_bytes ? t : tail_bytes - 1];
      v |= (t < tail_bytes ? byte : 0u) << (8 * k);
    }
    w[u] = v;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Slot of tile q (full or tail); `q`, `full_tiles` and `tail_bytes` are
// uniform across the wavefront, so the choice is a scalar branch.
__device__ __forceinline__ uint4 load_slot(const uint8_t* __restrict__ panel, int q,
                                           int full_tiles, int tail_bytes, int g, int r) {
  if (q < full_tiles) return load_full_slot(panel, q, g, r);
  return load_tail_slot(panel, full_tiles, tail_bytes, g, r);
}

// Workgroup barrier without a memory fence: this wavefront's LDS accesses
// complete, then s_barrier; the memory clobber keeps the compiler from moving
// memory accesses across it. (__syncthreads would also wait for every global
// load in flight, since the loader's LDS copies count as global loads.) LDS
// copies (global_load_lds) are waited for explicitly by the loader before
// the barrier that publishes them.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Index of the calling thread's wavefront as a wave-uniform (scalar) value,
// so that branches on it are scalar and do not make the compiler wait for
// outstanding loads at their joins.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Copy n (>= 1) elements from global memory to LDS with all of a thread's
// loads in flight before its first LDS store (PER loads per thread per
// round). The stores are unconditional: out-of-range ones go to dst[n],
// which must exist (one spare element).
template <int PER, typename T>
__device__ __forceinline__ void copy_to_lds(T* __restrict__ dst, const T* __restrict__ src, int n) {
  for (int base = 0; base < n; base += PER * (int)blockDim.x) {
    T v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = base + j * (int)blockDim.x + (int)threadIdx.x;
      v[j] = src[i < n ? i : n - 1];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = base + j * (int)blockDim.x + (int)threadIdx.x;
      dst[i < n ? i : n] = v[j];
    }
  }
}

// Cross-workgroup hand-off of split-K partial sums without whole-cache
// maintenance (an agent-scope fence would write back and invalidate the
// XCD's entire L2): the partials are written and read with device-coherent
// (agent-scope) relaxed atomic stores and loads, which go to the device
// coherence point instead of an XCD's L2. Every wave waits for its stores to
// complete (vmcnt 0) before the ticket is taken; compiler-level fences keep
// the loads after it.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Returns true in every thread of the workgroup that takes the last of
// `count` tickets of `ticket`. All partial stores of the workgroup must be
// issued before the call.
__device__ __forceinline__ bool last_ticket(unsigned* ticket, int count, int* flag) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0x0F70);   // gfx9 encoding: vmcnt(0), expcnt(7), lgkmcnt(15)
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            (unsigned)(count - 1);
  __syncthreads();
  const bool last = *flag != 0;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return last;
}

// Timing of the sign-product kernels (the C ABI's lq_profile_events): when
// a pair of events is pending for the calling thread, the next sign-product
// launch takes it, and the events are recorded by the dispatch itself at the
// kernel's start and end (hipExtLaunchKernelGGL), as a profiler times it.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();   // thread-local, defined with the C ABI

template <typename Kernel, typename... Args>
hipError_t launch_timed(Kernel kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                        Args... args) {
  LaunchEvents& ev = launch_events();
  if (ev.start != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, ev.start, ev.stop, 0u, args...);
    ev = LaunchEvents{};
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
// Every launcher enqueues on `stream` and returns hipGetLastError().

// Launch shapes of the product kernels that the plan query reports.
constexpr int kLargeWaves = 4;         // sign_mfma_large_kernel, wspace_kernel
constexpr int kWsPanelsPerWave = 4;    // wspace_kernel
constexpr int kChunkLoaders = 4;       // sign_fp6_chunked_kernel: loader wavefronts
constexpr int kValuWaves = 4;          // sign_valu_kernel (one panel per wavefront)
constexpr int kOneLaunchWaves = 8;     // decode_fused / decode_self / decode_split kernels
constexpr int kSplitPanels = 2 * kOneLaunchWaves;   // decode_split_kernel: panels per workgroup

hipError_t launch_pack(const int8_t* signs, int64_t N, int64_t L, uint8_t* packed,
                       hipStream_t stream);
hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t L, int8_t* signs,
                         hipStream_t stream);
hipError_t launch_hadamard_scale(const void* x, bool x_bf16, int64_t B, int64_t K, int hb,
                                 const float* c, float* xt, hipStream_t stream);
hipError_t launch_lift(const float* xt, int64_t B, int64_t K, int d, int D, const float* M,
                       void* z, bool z_bf16, hipStream_t stream);

// ---- small batch (B <= 16): activation preparation and sign products.
// VALU product: column ranges of a panel group are combined through a ticket
// counter per group (every workgroup writes partial sums, the last to take a
// ticket adds them); the tickets are cleared by the launch before it.

// Activation operand of the FP4 x FP6 product. Batch row b takes nt MFMA
// columns cc = b * nt + t (term t), grouped in sets of 16 (cs = cc / 16,
// c = cc % 16, ncs = columns in the set). Per full or tail tile one record
// of `rec` bytes:
//   data   [cs][u][g][c] 24 bytes: 6 dwords of FP6 E2M3 codes (code m at bit
//          6m, the value meeting reduction index k = 32g + m of MFMA u); set
//          cs starts at 384 * 16 * cs (blocks are 8-byte aligned)
//   scales [cs][g][c] dword at 384 * ncv + 256 * cs: byte u is the E8M0
//          scale of that 32-value block
//   tpart  [b] float at 400 * ncv: sum over the tile's plane-0..2 columns of
//          the values the terms represent
struct OperandShape {
  int nt;     // terms per batch row
  int ncv;    // columns (B * nt)
  int cs;     // 16-column sets
  int rec;    // bytes per tile record (multiple of 16)
};
constexpr int kAopBlockBytes = 24;
__host__ __device__ __forceinline__ int aop_data_offset(int cs, int u, int g, int c, int ncs) {
  return 384 * 16 * cs + ((u * 4 + g) * ncs + c) * kAopBlockBytes;
}
// bytes between the blocks of MFMA u and u + 1 of one column
__host__ __device__ __forceinline__ int aop_u_stride(int ncs) { return 4 * kAopBlockBytes * ncs; }
__host__ __device__ __forceinline__ int aop_scale_offset(int ncv, int cs, int g, int c, int ncs) {
  return 384 * ncv + 256 * cs + (g * ncs + c) * 4;
}
__host__ __device__ __forceinline__ int aop_tpart_offset(int ncv) { return 400 * ncv; }
// Store one block's six code dwords (8-byte aligned).
__device__ __forceinline__ void aop_store_block(uint8_t* p, const uint32_t* dw) {
  uint2* q = reinterpret_cast<uint2*>(p);
  q[0] = make_uint2(dw[0], dw[1]);
  q[1] = make_uint2(dw[2], dw[3]);
  q[2] = make_uint2(dw[4], dw[5]);
}

struct OperandPlan {
  OperandShape s;
  uint8_t* aop;   // ext_tiles records, then 1024 bytes of slack for chunked copies
};
OperandShape operand_shape(int64_t B, bool z_bf16);
size_t operand_bytes(int64_t L, const OperandShape& s);

// Small-batch product plan: a workgroup multiplies P panels over the whole
// row; the row's activation records either all sit in LDS (sign_fp6.hip)
// or stream through it in chunks (`chunked`, sign_fp6_chunked.hip).
struct Fp6Plan {
  bool chunked;
  bool stream;            // resident: each tile's record (<= 1 KB) loaded with its slots
  int p;                  // panels per workgroup
  int w;                  // wavefronts per workgroup (chunked: compute wavefronts, plus a loader)
  int pgroups;            // panel groups
  int groups;             // workgroups (= pgroups)
  int red_off;            // resident: LDS offset of the tail tile's slots (after the records)
  int tpc, nch, chunk_bytes;   // chunked: tiles per wavefront per chunk, chunks, LDS per chunk
  size_t lds_bytes;       // dynamic LDS per workgroup
};
// Chosen for one layer; panels_per_group 0: free; device_cus: compute units
// of the device (0: unknown, taken as 256).
Fp6Plan plan_fp6(int64_t B, const PackedGeom& g, const OperandShape& s, int device_cus,
                 int panels_per_group = 0);
// One plan for n layers launched together (same kernel and panels per
// workgroup), and each layer's share under it.
Fp6Plan plan_fp6_group(int64_t B, const PackedGeom* gs, int n, const OperandShape& s,
                       int device_cus);
Fp6Plan plan_fp6_layer(const Fp6Plan& group, const PackedGeom& g, const OperandShape& s);
// The chunked kernel's plan and instances (sign_fp6_chunked.hip).
bool fp6_records_fit(const PackedGeom& g, const OperandShape& s);
Fp6Plan plan_fp6_chunked(const PackedGeom& g, const OperandShape& s, int device_cus,
                         int panels_per_group);
void fill_chunks(Fp6Plan* p, const PackedGeom& g, const OperandShape& s);

// Fused decode (whitening, lift, operand and product in one launch; the
// operand record of each (tile, batch row) is produced by one workgroup and
// published through per-tile flags in the workspace's control area).
constexpr int kFusedCtlWords = 128;    // epoch, ticket, done, error words (128 B apart)
constexpr int kFusedErrorWord = 96;
constexpr int kMaxFusedTiles = 256;    // flags [tile][16] for at most this many column tiles
constexpr size_t kFusedControlBytes = (size_t)(kFusedCtlWords + kMaxFusedTiles * 16) * 4;
// The split one-launch decode's per-panel-group tickets follow.
constexpr int kSplitTickets = 1024;
constexpr size_t kControlBytes = kFusedControlBytes + (size_t)kSplitTickets * 4;
struct FusedPlan {
  bool ok;          // applicable (one column set, producers <= workgroups, LDS fits)
  int p, tpc, nch, chunk_bytes, groups, producers;
  size_t lds_bytes;
};
// `cus`: compute units of the device (all producers must be co-resident).
FusedPlan plan_fused(int64_t B, const PackedGeom& g, const OperandShape& s, int cus);
// Test aid: while set, the loaders of decode_fused launches wait for a
// publication no producer makes and give up after a few polls (the error
// word is set; every kernel still runs to its end).
void set_fused_forced_timeout(bool on);
hipError_t launch_decode_fused(const uint8_t* packed, const PackedGeom& g, const void* x,
                               bool x_bf16, int64_t B, int64_t K, int d, int D, int hb,
                               const float* c, const float* M, const OperandPlan& op,
                               unsigned* ctl, const float* row_scale, void* y, bool y_bf16,
                               const FusedPlan& plan, hipStream_t stream);

// One-launch decode split over the reduction (batch 1): workgroup (tile
// group, 16-panel group) prepares the operand of its tiles only; the tile
// groups' partial row sums meet through a ticket per panel group.
struct SplitPlan {
  bool ok;
  int tpg, kgroups, pgroups;   // tiles per group, tile groups, panel groups
  int xl;                      // x values per thread (2 per 1024-input chunk of the span)
  size_t lds_bytes, partial_bytes;
};
SplitPlan plan_split(int64_t B, int64_t K, int d, int D, const PackedGeom& g,
                     const OperandShape& s, int cus);
hipError_t launch_decode_split(const uint8_t* packed, const PackedGeom& g, const void* x,
                               bool x_bf16, int64_t K, int d, int D, int hb, const float* c,
                               const float* M, const OperandShape& s, const float* row_scale,
                               void* y, bool y_bf16, const SplitPlan& plan, float* partial,
                               unsigned* tickets, hipStream_t stream);

// One-launch decode without communication (batch 1, short rows): every
// workgroup prepares the whole operand in LDS and multiplies 8 panels.
struct SelfPlan {
  bool ok;
  int kx, groups, pw;   // K rounded up to 1024; workgroups; panels per workgroup
  size_t lds_bytes;
};
SelfPlan plan_self(int64_t B, int64_t K, int d, int D, const PackedGeom& g, const OperandShape& s);
hipError_t launch_decode_self(const uint8_t* packed, const PackedGeom& g, const void* x,
                              bool x_bf16, int64_t K, int d, int D, int hb, const float* c,
                              const float* M, const OperandShape& s, const float* row_scale,
                              void* y, bool y_bf16, const SelfPlan& plan, hipStream_t stream);

struct ValuPlan {
  int bt, tps, ksplit, groups;
  size_t partial_bytes;
};
ValuPlan plan_valu(int64_t B, const PackedGeom& g);

// Several layers that read the same x (same K) in one preparation launch and
// one product launch: at most this many.
constexpr int kMultiMax = 4;
// One layer of a preparation launch (kernel argument, by value).
struct PrepLayer {
  const float* c;
  const float* M;
  uint8_t* aop;
  int d, D, lhb, L;
  float norm;
  int tiles;        // its 512-column lifted tiles (workgroups along the grid's x dimension)
};
struct PrepTable {
  int n;
  PrepLayer l[kMultiMax];
};
// A layer of launch_prep_multi, as the caller describes it.
struct PrepLayerDesc {
  int d, D, hb;
  int64_t L;
  const float* c;
  const float* M;
  uint8_t* aop;     // its operand records (operand_bytes(L, s))
};
// The FP6 operands of n <= kMultiMax layers for the same x (bf16 or fp32).
hipError_t launch_prep_multi(const void* x, bool x_bf16, int64_t B, int64_t K, int n,
                             const PrepLayerDesc* layers, const OperandShape& s,
                             hipStream_t stream);

// xkind: 0 x fp32, 1 x bf16 (whiten + lift), 2 z fp32, 3 z bf16 (as given).
// op == nullptr: write fp32 z to zf32 (B x L); else the FP6 operand.
hipError_t launch_prep(const void* x, int xkind, int64_t B, int64_t K, int d, int D, int hb,
                       const float* c, const float* M, int64_t L, float* zf32,
                       const OperandPlan* op, unsigned* tickets, int n_tickets,
                       hipStream_t stream);
hipError_t launch_sign_fp6(const uint8_t* packed, const PackedGeom& g, const OperandPlan& op,
                           int64_t B, const float* row_scale, void* y, bool y_bf16,
                           const Fp6Plan& plan, hipStream_t stream);
// One layer of a small-batch product launch (kernel argument, by value).
struct SignLayer {
  const uint8_t* packed;
  const uint8_t* aop;
  const float* row_scale;
  void* y;
  int64_t panel_bytes;
  int panels, full_tiles, tail_bytes, N;
  int nch;             // chunked kernel: chunks of full tiles
  int group_begin;     // its first workgroup
};
struct SignTable {
  int n;
  SignLayer l[kMultiMax];
};
// A layer of launch_sign_fp6_multi: its geometry, operand, outputs and the
// plan a call of its own would use.
struct SignLayerDesc {
  const uint8_t* packed;
  PackedGeom g;
  const uint8_t* aop;
  const float* row_scale;
  void* y;
  Fp6Plan plan;
};
// Whether two layers' plans can share one launch (same kernel instance).
bool fp6_plans_match(const Fp6Plan& a, const Fp6Plan& b);
hipError_t launch_sign_fp6_multi(int n, const SignLayerDesc* layers, const OperandShape& s,
                                 int64_t B, bool y_bf16, hipStream_t stream);
hipError_t launch_fp6_chunked_table(const SignTable& tab, int groups, const OperandShape& s,
                                    int64_t B, bool y_bf16, const Fp6Plan& plan,
                                    hipStream_t stream);
hipError_t launch_sign_valu(const uint8_t* packed, const PackedGeom& g, const void* z,
                            bool z_bf16, int64_t B, const float* row_scale, void* y, bool y_bf16,
                            const ValuPlan& plan, float* partial, unsigned* tickets,
                            hipStream_t stream);
hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t stream);

// ---- large batch: bf16 matrix-core GEMM (z bf16, or fp32 as a hi + lo pair).
// z is first rewritten into the operand order of the product ("zp": per 16
// batch rows and 128-column step a 4 KB block; nterm bf16 planes).
struct ZpGeom {
  int64_t B16, steps;
  int nterm;
  size_t bytes;        // zp itself
  size_t tail_bytes;   // the tail tile's slots in full-tile form (1 KB per panel), if L % 512
};
ZpGeom zp_geom(int64_t B, const PackedGeom& g, bool z_bf16);
struct LargePlan {
  int ppw, jb;      // panels per compute wavefront, 16-row batch tiles per workgroup
  int ksplit, tps;  // reduction ranges (1: none) and tiles per range
  size_t partial_bytes;   // ksplit > 1: fp32 partial sums, ksplit x B x N
};
LargePlan plan_large(int64_t B, const PackedGeom& g, bool z_bf16);
// kind 0: z fp32, 1: z bf16 (both B x L); 2: lift xt (B x K fp32) with M into
// fp32-precision zp (two planes), 3: the same into bf16 zp (one plane).
hipError_t launch_zp(const void* src, int kind, int64_t B, int64_t L, int64_t K, int d, int D,
                     const float* M, const PackedGeom& g, void* zp, hipStream_t stream);
// partial: LargePlan::partial_bytes of workspace (unused when ksplit is 1).
hipError_t launch_sign_mfma_large(const uint8_t* packed, const PackedGeom& g, const void* zp,
                                  void* tail_slots, bool z_bf16, int64_t B,
                                  const float* row_scale, void* y, bool y_bf16, float* partial,
                                  hipStream_t stream);
// The tail tile's slots of every panel in full-tile form (1 KB per panel;
// columns past L read as +1 signs).
hipError_t launch_tail_slots(const uint8_t* packed, const PackedGeom& g, void* out,
                             hipStream_t stream);

// ---- large batch in W space: the dense weights rebuilt per block from the
// signs (a table of the 2^D sign patterns' weight vectors), bf16 MFMAs over
// K' = d Kb. D in {4, 8} (whole blocks per packed word), d <= 4.
bool wspace_supported(int d, int D);
struct XpGeom {
  int64_t B16, steps;
  size_t bytes;        // xp: per 16 batch rows and step (8 blocks per lane), d KB
  size_t tail_bytes;   // as ZpGeom
};
XpGeom xp_geom(int64_t B, const PackedGeom& g, int d, int D);
int plan_wspace_jb(int64_t B, const PackedGeom& g, int d);   // 16-row batch tiles per workgroup
// ---- nearest-neighbour encoding and the training step of M (encode.hip)
constexpr int kEncodeMaxD = 24;        // exhaustive search: 2^D sign vectors per block
constexpr int kEncodePinvMaxD = 32;    // pseudo-inverse search: D
constexpr int kEncodePinvMaxFree = 24; // ... and 2^(D - d) sign vectors per block
constexpr int kEncodeMaxSmallD = 16;   // d (the residual lives in registers)
constexpr int kTrainMaxD = 24;
hipError_t launch_encode(const float* w, int64_t nblocks, int d, int D, const float* M,
                         int8_t* signs, float* dist2, hipStream_t stream);
// AB: device doubles, A = M_a^-1 (d x d, row-major) then A M_f (d x (D - d), row-major).
hipError_t launch_encode_pinv(const float* w, int64_t nblocks, int d, int D, const float* M,
                              const double* AB, int8_t* signs, float* dist2, hipStream_t stream);
int train_groups(int64_t n);
size_t train_workspace_bytes(int64_t n, int d, int D);
hipError_t launch_train_step(float* M, const float* w, int64_t n, int d, int D, float lr,
                             float* loss, void* ws, hipStream_t stream);

// Whitening of x straight into xp (no xt in memory).
hipError_t launch_xpw(const void* x, bool x_bf16, int64_t B, int64_t K, int hb, const float* c,
                      int d, int D, const PackedGeom& g, void* xp, hipStream_t stream);
hipError_t launch_wspace(const uint8_t* packed, const PackedGeom& g, const void* xp,
                         void* tail_slots, int64_t B, const float* M, int d, int D,
                         const float* row_scale, void* y, bool y_bf16, hipStream_t stream);

}  // namespace lq
