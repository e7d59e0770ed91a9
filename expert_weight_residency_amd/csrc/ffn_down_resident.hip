// Down GEMM for decode-sized steps as a persistent, continuously streaming
// kernel (gfx950). Same operation as the down kernels in ffn_mxfp4.hip and
// ffn_tiled.hip: Y[s][o] = bf16(Wdown[r][o] . h[s]) for every slot s routed to
// active row r ("vLLM: Pin Hot Experts", section "Results, September 17": the
// routed MXFP4 expert FFN per bank, unweighted rows for a later finalize).
//
//  - One workgroup of 8 wavefronts per CU (for a device bank on all CUs but
//    the few a host-bank launch beside it holds; for a bank in host memory on
//    those few). Work item = kNG groups of 16 output rows of one active expert.
//    Items are ordered (expert, row block); workgroup b takes one contiguous
//    run of them (equal runs over all workgroups, so every CU has work), so a
//    workgroup touches one or two experts (a few at small H), and its
//    wavefronts take the run's items one at a time from a counter in LDS. (A
//    SIMD issues for its oldest wavefront first: with fixed equal shares (16
//    wavefronts per CU at the time) its wavefronts finished one after another,
//    ~47, 68, 93 and 105 us into a decode step, the last quarter of the time
//    with a quarter of the loads in flight. Taking items as they go, the
//    wavefronts finish within about one item of each other.)
//  - The down GEMM's B operand is h, one row per slot, so unlike gate/up the
//    activations are not shared by every workgroup. Each workgroup stages the
//    h rows of the slots of its experts into LDS (zero-padded to whole
//    chunks) behind one barrier; if they do not fit, it runs phases of as many
//    rows as fit, and an item's weights are streamed once per phase holding
//    some of its slots.
//  - Each wavefront then streams its items' weight chunks back to back, a few
//    ahead in a register ring, across item boundaries; only weight loads and
//    one scale-block load per item go through the vector-memory queue. Each
//    chunk of a 16-row item is read as two whole-line loads (rows 0-7, rows
//    8-15) and the halves are exchanged between partner lanes (see
//    mxfp4_common.h). For a bank in HBM whose rows allow it, every load reads
//    one aligned 128-byte line with the streaming cache policy, and each
//    chunk is put together on chip from two of them (see kAligned below).
//  - An item's scale bytes (16 * kNG rows x I/32 bytes) are contiguous and
//    16-byte aligned: the wavefront loads them with a few 16-byte loads when
//    its prefetch enters the item, copies them into its own LDS slot when it
//    starts the item, and reads each chunk's pair from there. (A 2-byte load
//    per chunk costs a whole memory instruction, and those instructions, not
//    bytes, bound these kernels; the 90-byte scale rows of I = 2880 also rule
//    out the 8-byte loads the gate/up kernel uses.)
//  - The last chunk of a reduction axis that is not a multiple of 256 has
//    lanes past the end: they read that chunk's first block with unit scale
//    and meet the zero padding of the staged h rows (the other kernel
//    families read the row's first block instead; finite values times zero,
//    accumulated from +0, give the same bits either way).
//  - Each output element sees the same MFMA sequence as in the other kernel
//    families (same 256-element chunks, same lane-to-element map, same order
//    from zero) and the same rounding, so a pick gives the same bits.
#include <algorithm>

#include "internal.h"
#include "mxfp4_common.h"

namespace moe {
namespace {

using namespace mx;

// 8 wavefronts. Unaligned loads, 2 chunks each in flight: a sweep of the
// decode step at H = 4096, I = 2880 (hot bank alone, us per launch;
// wavefronts x chunks): 16x5 92.8, 16x2 90.1, 12x5 91.5, 12x2 89.6, 10x2 89.3,
// 8x5 88.4, 8x3 87.4, 8x2 86.2, 8x1 86.3, 6x3 86.0, 6x2 85.6, 4x5 94.8, 4x11
// 96.6, 8x11 91.8: more requests in flight than the CU needs to keep its
// share of HBM busy only evict, between the two chunks that read it, the line
// a 1440-byte row shares with its neighbour (with the streaming cache policy
// 16x5 takes 104.9). Aligned streaming loads (each line read once), 3 chunks
// in flight, in an A/B against the unaligned kernel's 83.6: 8x3 78.3-78.7,
// 12x3 78.2, 16x3 78.3, 16x2 77.9, 8x2 83.2, 8x5 78.8, 8x11 83.0, 6x3 88.9;
// aligned with the ordinary cache policy, 8x2: 85.0.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kNG = 1;    // 16-row MFMA groups per item
constexpr int kP = 2;     // weight chunks in flight per wavefront (ring of kP + 1)
constexpr int kPAl = 3;   // the same with line-aligned loads
constexpr int kSbl = 2;   // 16-byte scale granules per lane per item (covers I <= 4096 / kNG)
constexpr size_t kLdsMax = 160 * 1024;  // gfx950: the LDS of one CU

struct Shape {
  int nchunk, kpad, sbr, sbw;  // chunks, padded axis, scale bytes per row / per item
};

__host__ __device__ inline Shape shape_of(int I) {
  Shape s;
  s.nchunk = (I + kChunkElems - 1) / kChunkElems;
  s.kpad = s.nchunk * kChunkElems;
  s.sbr = I / 32;
  s.sbw = kNG * 16 * s.sbr;
  return s;
}

// LDS: h rows [max_rows][kpad] bf16 | per-wavefront scale slots [kWaves][sbw] |
// slot ids of the staged rows [max_rows].
__host__ __device__ inline size_t lds_bytes(const Shape& s, int max_rows) {
  return (size_t)max_rows * s.kpad * 2 + (size_t)kWaves * s.sbw + (size_t)max_rows * 4;
}

// kAligned: every weight load reads whole aligned lines. Rows of I/2 bytes
// start m = (row * I/2) mod 128 bytes into a line (0, 32, 64 or 96 at
// I = 2880), so the operand layout's chunk c of a row (128 bytes from the row
// start) straddles two lines, and a line is read once by each of the two
// chunks that share it (twice the line requests, and the line at a row
// boundary is read again a row later). Instead load c of a row reads the
// row's c-th aligned line (from the row start rounded down), and chunk c is
// put together on chip from loads c and c + 1: lane piece p (16 bytes) takes
// piece p + m/16 of the two lines' concatenation. The source lane of that
// piece sends load c's value if the piece lies in the first line, else load
// c + 1's, and one ds_bpermute per dword moves it; the lanes then hold exactly
// the bytes the unaligned loads would give (same MFMA inputs, same bits). The
// last chunk needs only load c when m + (its bytes) <= 128 for every row,
// which the launcher checks (an item's 16 rows are line-aligned as a whole
// when the tensor is, so its last row's last line ends at the item's end and
// its first row's first line starts at the item's start: no load leaves the
// item). Each line is then read by one load (but the line a row ends in and
// the next row starts in, read by both rows about one item apart), so the
// loads take the streaming cache policy (78 against 84 us per decode step
// with the unaligned loads).
template <bool kAligned>
__global__ __launch_bounds__(kThreads, 1) void ffn_down_resident(
    const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ active_rows,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots,
    const __bf16* __restrict__ h, int H, int I, int max_rows, uint16_t* __restrict__ Y) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Shape sh = shape_of(I);
  const int nchunk = sh.nchunk, kpad = sh.kpad, sbr = sh.sbr;
  const int nblk = I / 32;
  __bf16* hs = reinterpret_cast<__bf16*>(smem);
  unsigned char* sc_all = smem + (size_t)max_rows * kpad * 2;
  int* l_slot = reinterpret_cast<int*>(sc_all + (size_t)kWaves * sh.sbw);

  const int tid = threadIdx.x;
  const int na = __builtin_amdgcn_readfirstlane(*n_active);
  const int per = H / (16 * kNG);  // items per expert
  const int n = na * per;
  if (n == 0) return;
  const int qb = (n + gridDim.x - 1) / gridDim.x;  // items per workgroup
  const int g0 = blockIdx.x * qb;
  if (g0 >= n) return;  // the whole workgroup, before any barrier
  const int g1 = min(n, g0 + qb);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  __shared__ int l_next;  // next item of the workgroup's run not yet taken
  const int s_lo = __builtin_amdgcn_readfirstlane(row_off[g0 / per]);
  const int s_hi = __builtin_amdgcn_readfirstlane(row_off[(g1 - 1) / per + 1]);

  const int lane = tid & 63, r = lane & 15, q = lane >> 4;
  const size_t wrb = I / 2;
  unsigned char* sc = sc_all + (size_t)wv * sh.sbw;  // this wavefront's scale slot
  const int ngran = sh.sbw / 16;

  for (int ph0 = s_lo; ph0 < s_hi; ph0 += max_rows) {
    const int ph1 = min(s_hi, ph0 + max_rows);
    if (ph0 != s_lo) __syncthreads();  // the previous phase is done with the rows
    {
      const int gpr = kpad / 8, nr = ph1 - ph0;
      for (int gi = tid; gi < nr * gpr; gi += kThreads) {
        const int m = gi / gpr, g = gi - m * gpr;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (g * 8 < I)
          v = *reinterpret_cast<const uint4*>(h + (size_t)slots[ph0 + m] * I + g * 8);
        *reinterpret_cast<uint4*>(hs + lds_elem(m, kpad, g * 8)) = v;
      }
      for (int i = tid; i < nr; i += kThreads) l_slot[i] = slots[ph0 + i];
      if (tid == 0) l_next = g0;  // every phase walks the whole run again
    }
    __syncthreads();

    // Slot positions of expert a inside this phase, and its 16-column passes.
    auto lo_of = [&](int a) {
      return max(__builtin_amdgcn_readfirstlane(row_off[a]), ph0);
    };
    auto ncols = [&](int a) {
      return min(__builtin_amdgcn_readfirstlane(row_off[a + 1]), ph1) - lo_of(a);
    };
    auto passes_of = [&](int it) {
      const int c = ncols(it / per);
      return c > 0 ? (c + 15) >> 4 : 0;
    };
    // The next item of the run with slots in this phase, or g1 when none is
    // left. One lane takes it from the counter; the value is wave-uniform.
    auto take = [&]() {
      int nx;
      do {
        int v = 0;
        if (lane == 0) v = atomicAdd(&l_next, 1);
        nx = __builtin_amdgcn_readfirstlane(v);
      } while (nx < g1 && passes_of(nx) == 0);
      return nx < g1 ? nx : g1;
    };
    int p_it = take();
    if (p_it >= g1) continue;  // the run is already taken

    // Prefetch cursor: item, pass, chunk, this lane's weight row, and the
    // item's scale block.
    int p_pass = 0, p_c = 0, p_np = passes_of(p_it);
    const uint8_t* pw;  // the item's first row (whole-line loads add this lane's offsets)
    const uint8_t* psb;
    auto p_enter = [&](int it) {
      const int a = it / per, o0 = (it - a * per) * 16 * kNG;
      const size_t row = (uint32_t)__builtin_amdgcn_readfirstlane(active_rows[a]);
      pw = w2 + (row * H + o0) * wrb;
      psb = s2 + (row * H + o0) * sbr;
    };
    p_enter(p_it);
    // Move the cursor from the end of a pass to the start of the next pass or
    // of the next item it takes. nchunk is a multiple of the ring length
    // kP + 1, so this happens at one fixed ring position (first step of a
    // pass's last cycle); everywhere else the cursor only steps to the next
    // chunk. When no item is left the cursor moves to the bank's first item
    // (p_it unchanged tells the consumer to stop): the few loads still issued
    // after that (fewer than nchunk) are never used, and every wavefront's
    // read the same lines, which stay in the L2 (re-reading the wavefront's
    // own last item, just streamed past the L2, fetched ~12 MB per launch).
    auto p_rollover = [&]() {
      p_c = 0;
      if (p_pass + 1 < p_np) {  // next 16 slots of the same item: its weights again
        ++p_pass;
        return;
      }
      const int nx = take();
      if (nx < g1) {
        p_pass = 0;
        p_it = nx;
        p_np = passes_of(nx);
        p_enter(nx);
      } else {
        pw = w2;  // the bank's first item, which every wavefront's last loads share
      }
    };
    // Whole-line loads (line_load_a/_b): lane r's partner r^8 has the same q,
    // so both are in range or both past the end of the axis. Only the last
    // chunk can have lanes past its end: they read inside that chunk's first
    // block (in the same cache line as the lanes in range); their scale is
    // replaced by unit and their activations are the zero padding, so what
    // they read does not change a bit of the result (finite E2M1 values times
    // zero, accumulated from +0).
    const bool upper = r >= 8;
    const bool lane_in_last = (nchunk - 1) * kChunkBlocks + 2 * q < nblk;
    // kAligned: rows 8 + r and r start equally far into a line (8 rows are
    // 8 * I/2 bytes, a multiple of 128)
    const uint32_t mis = kAligned ? (uint32_t)(((size_t)(r & 7) * wrb) & 127u) : 0u;
    const size_t off_a = line_load_a(r, q, wrb) - mis, off_b = line_load_b(r, q, wrb) - mis;
    const size_t last_a =
        (nchunk - 1) * 128 + (kAligned || lane_in_last ? off_a : off_a - 32 * q);
    const size_t last_b =
        (nchunk - 1) * 128 + (kAligned || lane_in_last ? off_b : off_b - 32 * q);
    // kAligned: this lane's 16-byte piece of its row in loads A and B, the
    // shift in pieces, whether the piece it holds is passed on from load c
    // (else from load c + 1), and the lane holding the piece it needs
    const int shift = (int)(mis >> 4);
    const int pa_me = 2 * q + (r >= 8 ? 1 : 0), pb_me = 2 * q + (r < 8 ? 1 : 0);
    const bool send_first_a = pa_me >= shift, send_first_b = pb_me >= shift;
    const int pa_src = (pa_me + shift) & 7, pb_src = (pb_me + shift) & 7;
    const int addr_a = ((r & 7) + 8 * (pa_src & 1) + 16 * (pa_src >> 1)) * 4;
    const int addr_b = ((r & 7) + 8 * (1 - (pb_src & 1)) + 16 * (pb_src >> 1)) * 4;
    auto realign = [&](const AChunk& first, const AChunk& second) {
      AChunk o;
      auto mv = [&](uint32_t x, uint32_t y, bool f, int addr) {
        return (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(f ? x : y));
      };
      o.lo.x = mv(first.lo.x, second.lo.x, send_first_a, addr_a);
      o.lo.y = mv(first.lo.y, second.lo.y, send_first_a, addr_a);
      o.lo.z = mv(first.lo.z, second.lo.z, send_first_a, addr_a);
      o.lo.w = mv(first.lo.w, second.lo.w, send_first_a, addr_a);
      o.hi.x = mv(first.hi.x, second.hi.x, send_first_b, addr_b);
      o.hi.y = mv(first.hi.y, second.hi.y, send_first_b, addr_b);
      o.hi.z = mv(first.hi.z, second.hi.z, send_first_b, addr_b);
      o.hi.w = mv(first.hi.w, second.hi.w, send_first_b, addr_b);
      return o;
    };
    // Unaligned loads take the ordinary cache policy: rows of I/2 bytes are
    // not line-aligned, so a line holding the end of one chunk and the start
    // of the next is read by two loads a chunk apart, and with the streaming
    // policy it is gone by the second (measured: whole-line loads 115 -> 102
    // us per decode step with the ordinary policy, no gain with the streaming
    // one). The scheduling barrier pins the loads at their place in the
    // stream (left free, the compiler sinks them towards the end of a ring
    // cycle, which shortens how far ahead they run).
    auto load_w = [&](AChunk& a) {
      const bool last = p_c == nchunk - 1;
      if constexpr (kAligned) {
        a.lo = ld_stream16(pw + (last ? last_a : p_c * 128 + off_a));
        a.hi = ld_stream16(pw + (last ? last_b : p_c * 128 + off_b));
      } else {
        a.lo = *reinterpret_cast<const uint4*>(pw + (last ? last_a : p_c * 128 + off_a));
        a.hi = *reinterpret_cast<const uint4*>(pw + (last ? last_b : p_c * 128 + off_b));
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // The scale block of the cursor's item, kSbl granules per lane (separate
    // variables: an array here ends up in scratch). Loaded at fixed points of
    // the stream, never under a condition, so that the compiler can count the
    // loads issued after it and waiting for it never waits for newer ones.
    uint4 sblk0, sblk1;
    // The scheduling barrier keeps the compiler from moving other loads
    // ahead of it.
    auto load_sblk = [&]() {
      sblk0 = *reinterpret_cast<const uint4*>(psb + 16 * (lane < ngran ? lane : 0));
      sblk1 = *reinterpret_cast<const uint4*>(psb + 16 * (lane + 64 < ngran ? lane + 64 : 0));
      __builtin_amdgcn_sched_barrier(0);
    };

    constexpr int P = kAligned ? kPAl : kP;
    AChunk ring[P + 1];
    load_sblk();
#pragma unroll
    for (int p = 0; p < P; ++p) {
      load_w(ring[p]);
      ++p_c;  // P < nchunk
    }

    // The items the cursor took, and their passes, in order; nchunk is a
    // multiple of kP + 1, so every pass starts at ring slot 0. In the last
    // ring cycle of a pass the cursor, after its first advance, stands at the
    // first chunk of the next pass or item: the scale block loaded there is
    // the one the next pass uses (the same block again when the next pass is
    // of the same item).
    for (int it = p_it;;) {
      const int np = passes_of(it);
      const int a = it / per, o0 = (it - a * per) * 16 * kNG;
      const int lo = lo_of(a), nt = ncols(a);
      for (int pass = 0; pass < np; ++pass) {
        if (pass == 0) {
          // the item's scale block: registers -> this wavefront's LDS slot
          // (lanes past the block hold granule 0, loaded from the clamped
          // address, and write it back to granule 0: no branch, same bytes)
          *reinterpret_cast<uint4*>(sc + 16 * (lane < ngran ? lane : 0)) = sblk0;
          *reinterpret_cast<uint4*>(sc + 16 * (lane + 64 < ngran ? lane + 64 : 0)) = sblk1;
          __builtin_amdgcn_wave_barrier();
        }
        const int j = pass * 16 + r;
        const bool has = j < nt;
        const int lrow = (has ? lo + j : lo) - ph0;  // staged h row of this column
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        // One loop body for every ring cycle (a separate copy for the last
        // cycle would keep the ring in other registers, and moving them
        // between copies waits for every load in flight).
        for (int c = 0; c < nchunk; c += P + 1) {
#pragma unroll
          for (int u = 0; u <= P; ++u) {
            const int cc = c + u;
            load_w(ring[(u + P) % (P + 1)]);
            if (u == 0 && c + P + 1 == nchunk) {
              p_rollover();
              load_sblk();
            } else {
              ++p_c;
            }
            const bool ok = cc != nchunk - 1 || lane_in_last;
            const uint32_t raw =
                *reinterpret_cast<const uint16_t*>(sc + (ok ? r * sbr + cc * 8 + 2 * q : 0));
            const uint32_t b = ok ? raw : 0x7f7fu;
            const float s0 = e8m0_to_f32(b & 0xffu), s1 = e8m0_to_f32(b >> 8);
            const int e0 = cc * kChunkElems + 64 * q;
            AChunk wc;
            if constexpr (kAligned)
              wc = realign(ring[u], ring[(u + 1) % (P + 1)]);
            else
              wc = ring[u];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
              const bf16x8 bv =
                  *reinterpret_cast<const bf16x8*>(hs + lds_elem(lrow, kpad, e0 + 8 * m));
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  dequant8(own_word(wc, m, upper), m < 4 ? s0 : s1), bv, acc, 0, 0, 0);
            }
          }
        }
        // lane (r, q) holds output rows o0 + 4q + v of the pass's column r
        if (has) {
          const size_t sl = (uint32_t)l_slot[lrow];
          uint32_t yb[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) yb[v] = f32_to_bf16_bits(acc[v]);
          *reinterpret_cast<uint2*>(Y + sl * H + o0 + 4 * q) =
              make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
        }
      }
      if (p_it == it) break;  // the cursor found no further item
      it = p_it;
    }
  }
}

// Rows of h one workgroup can stage, at most `want` (the kernel's static LDS,
// the item counter, is kept out of the dynamic allocation's budget).
constexpr size_t kStaticLds = 256;
int rows_that_fit(const Shape& s, int want) {
  const size_t dev = device_lds_per_block();
  const size_t lim = (dev < kLdsMax ? dev : kLdsMax) - kStaticLds;
  const size_t fixed = (size_t)kWaves * s.sbw;
  if (fixed >= lim) return 0;
  const size_t per_row = (size_t)s.kpad * 2 + 4;
  const size_t fit = (lim - fixed) / per_row;
  return (int)(fit < (size_t)want ? fit : (size_t)want);
}

}  // namespace

namespace {
// Line-aligned loads (device banks): the weight tensor 128-byte aligned, so
// that every item starts on a line, and the last chunk's bytes of every row
// inside the row's last aligned line, m + (I/2 - 128 (nchunk - 1)) <= 128 for
// each row's offset m into its first line; whole ring turns per pass.
bool down_aligned(int I, const void* w2, int on_host) {
  const Shape s = shape_of(I);
  const int wrb = I / 2, last = wrb - 128 * (s.nchunk - 1);
  int mmax = 0;
  for (int r = 0; r < 8; ++r) mmax = std::max(mmax, (r * wrb) & 127);
  return !on_host && (reinterpret_cast<uintptr_t>(w2) & 127u) == 0 && mmax + last <= 128 &&
         s.nchunk % (kPAl + 1) == 0;
}
}  // namespace

bool ffn_use_down_resident(int T, int k, int H, int I, const void* w2, const void* s2,
                           int on_host) {
  const Shape s = shape_of(I);
  return T >= 1 && I % 32 == 0 && H % (16 * kNG) == 0 &&
         (s.nchunk % (kP + 1) == 0 || down_aligned(I, w2, on_host)) &&
         (reinterpret_cast<uintptr_t>(w2) & 15u) == 0 &&
         s.sbw % 16 == 0 && s.sbw <= kSbl * 64 * 16 &&
         (reinterpret_cast<uintptr_t>(s2) & 15u) == 0 && rows_that_fit(s, T * k) >= 1;
}

hipError_t launch_down_resident(const uint8_t* w2, const uint8_t* s2, int cap, int on_host,
                                const moe_split& sp, int T, int k, int H, int I,
                                const uint16_t* h_ws, uint16_t* Y, hipStream_t stream) {
  (void)cap;
  const Shape s = shape_of(I);
  const int max_rows = rows_that_fit(s, T * k);
  const int cus = device_cus();
  const int grid = on_host ? kHostBankCUs : (cus > 2 * kHostBankCUs ? cus - kHostBankCUs : cus);
  auto kern = down_aligned(I, w2, on_host) ? ffn_down_resident<true> : ffn_down_resident<false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds_bytes(s, max_rows), stream, w2, s2,
                     sp.n_active, sp.active_rows, sp.row_off, sp.slots,
                     reinterpret_cast<const __bf16*>(h_ws), H, I, max_rows, Y);
  return hipGetLastError();
}

}  // namespace moe
