// Gate/up + SwiGLU for decode-sized steps with the activations resident in LDS
// (gfx950). Same operation as the gate/up kernels in ffn_mxfp4.hip and
// ffn_tiled.hip ("vLLM: Pin Hot Experts", section "Results, September 17":
// the routed MXFP4 expert FFN per bank), organised so that a wavefront's
// weight stream never drains:
//
//  - One workgroup of 8 wavefronts per CU: for a device bank on all CUs but
//    the few a host-bank launch beside it holds, for a bank in host memory on
//    those few. It stages every token row of x
//    (T <= 16 rows of H) and the split's bookkeeping (active rows, offsets,
//    the token of every slot) into LDS once, behind one barrier; each
//    wavefront issues its first item's weight loads before that, so the
//    staging and the first weights share one round trip to memory (162 vs
//    164 µs per decode step). After that no wavefront waits for another.
//  - Work item = 16 i-columns of one active expert (its 16 gate rows and 16
//    up rows). Workgroup b owns one equal contiguous run of items, and its
//    wavefronts take the run's items one at a time from a counter in LDS (a
//    SIMD serves its oldest wavefront first, so fixed equal shares finish
//    one after another and leave the last part of the launch with few loads
//    in flight). Each wavefront streams its items' weight chunks back to
//    back, kP chunks ahead in a register ring, so the prefetch runs straight
//    across item boundaries. Inside the loop the global loads are the weight
//    chunks, issued unconditionally (past the wavefront's last chunk it
//    reads 4 chunks of the bank's first rows, shared by every wavefront and
//    held in the L2), so waiting for one chunk
//    never waits for a newer one, and the scale lines of each item the
//    prefetch enters.
//  - Each chunk of a 16-row group is read as two whole-line loads (rows 0-7,
//    rows 8-15) with the streaming cache policy, and the halves are
//    exchanged between partner lanes (see mxfp4_common.h): 163 -> 148 us
//    alone per decode step against the two half-line loads of the operand
//    layout (the gate/up rows of H/2 = 2048 bytes are line-aligned).
//  - Each row's scale bytes (one 128-byte line at H = 4096) are loaded once
//    per item, 32 bytes per lane (the row's four lanes hold the whole line),
//    and every 4 chunks each lane's pairs are taken from the line with
//    ds_bpermute and redistributed across the lane quarters with two
//    lane-swap instructions. A per-chunk 2-byte load per lane cost a whole
//    memory instruction for 1/16 of the bytes (those instructions, not the
//    bytes, bounded the first version: 197 -> 164 us per decode step with 8
//    bytes per lane per 4 chunks); reading the line in four such pieces, ~9
//    us apart, let the L2 drop it in between (1.07x the algorithmic bytes).
//    Holding the whole line takes the registers of 8 wavefronts per CU rather
//    than 16: 142.3 -> 137.5 us per decode step (16 wavefronts with quarter
//    lines against 8 with whole lines; 12 with whole lines 138.6).
//  - An item's tokens are the MFMA columns (16 per pass; an expert with more
//    than 16 slots, which needs duplicate ids in a token, takes more passes).
//  - Each output element sees the same MFMA sequence as in the other kernel
//    families (same 256-element chunks, same lane-to-element map, same order
//    from zero) and the same SwiGLU, so a pick gives the same bits.
#include "internal.h"
#include "mxfp4_common.h"

namespace moe {
namespace {

using namespace mx;

constexpr int kWaves = 8;                // wavefronts per workgroup (one workgroup per CU)
constexpr int kThreads = 64 * kWaves;
constexpr int kNG = 2;                   // MFMA row groups per item (gate, up)

// Bytes of LDS the kernel needs: activations, then int32 tables.
size_t resident_lds_bytes(int T, int k, int H, int cap) {
  const size_t kpad = (size_t)(H + kChunkElems - 1) / kChunkElems * kChunkElems;
  return (size_t)T * kpad * sizeof(uint16_t) +
         ((size_t)cap + (size_t)cap + 1 + 2 * (size_t)T * k) * sizeof(int32_t);
}

// Chunk c of a 16-row group as two whole-line loads (lo = load A, hi = load
// B; see line_load_a/_b): pa, pb point at this lane's two offsets of chunk 0.
__device__ __forceinline__ void load_w(AChunk& a, const uint8_t* __restrict__ pa,
                                       const uint8_t* __restrict__ pb, int c) {
  a.lo = ld_stream16(pa + c * 128);
  a.hi = ld_stream16(pb + c * 128);
}



// Lane (r, q) holds raw = the 8 scale bytes of chunk c0 + q of its row r
// (pair j = bytes 2j, 2j+1 belongs to lane quarter j). Transpose the 4 x 4
// pairs across the four lane quarters (lanes r, r+16, r+32, r+48): afterwards
// lane (r, q) holds its own pair of chunks c0 .. c0+3 as x.lo, y.lo, x.hi,
// y.hi. permlane32_swap(a, b) exchanges a's lanes 32-63 with b's lanes 0-31;
// permlane16_swap(a, b) exchanges a's odd 16-lane rows with b's even rows.
__device__ __forceinline__ void scale_quad(uint2 raw, uint32_t& x, uint32_t& y) {
  const auto h = __builtin_amdgcn_permlane32_swap(raw.x, raw.y, false, false);
  const uint32_t lo = h[0], hi = h[1];
  const uint32_t px = __builtin_amdgcn_perm(hi, lo, 0x05040100u);  // lo.low16, hi.low16
  const uint32_t py = __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // lo.high16, hi.high16
  const auto v = __builtin_amdgcn_permlane16_swap(px, py, false, false);
  x = v[0];
  y = v[1];
}

// The 8 scale bytes of chunk c0 + q of this lane's row (the layout scale_quad
// takes), from the row's whole 128-byte scale line held across the row's four
// lanes: lane (r, q) holds bytes 32q .. 32q+31 (chunks 4q .. 4q+3) in blk, so
// quad Q's piece q sits in lane (r, Q), dwords 2q and 2q+1.
__device__ __forceinline__ uint2 quad_from_line(const uint4 (&blk)[2], int r, int q, int Q) {
  const int src = (r + 16 * Q) << 2;
  const uint32_t w[8] = {blk[0].x, blk[0].y, blk[0].z, blk[0].w,
                         blk[1].x, blk[1].y, blk[1].z, blk[1].w};
  uint32_t v[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) v[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)w[d]);
  const uint32_t x = q == 0 ? v[0] : (q == 1 ? v[2] : (q == 2 ? v[4] : v[6]));
  const uint32_t y = q == 0 ? v[1] : (q == 1 ? v[3] : (q == 2 ? v[5] : v[7]));
  return make_uint2(x, y);
}

template <int P>
__global__ __launch_bounds__(kThreads, 2) void ffn_gate_up_resident(
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ s13,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ active_rows,
    const int32_t* __restrict__ row_off, const int32_t* __restrict__ slots,
    const __bf16* __restrict__ x, int T, int k, int H, int I, uint16_t* __restrict__ h_ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int kpad = (H + kChunkElems - 1) / kChunkElems * kChunkElems;
  __bf16* xs = reinterpret_cast<__bf16*>(smem);
  const int na = *n_active;
  int* l_rows = reinterpret_cast<int*>(xs + (size_t)T * kpad);  // [na]
  int* l_off = l_rows + na;                                     // [na + 1]
  int* l_slot = l_off + na + 1;                                 // [T*k] slot ids, split order
  int* l_tok = l_slot + T * k;                                  // [T*k] their tokens

  const int tid = threadIdx.x;
  const int picks = T * k;
  const int per = I / 16;  // items per expert
  const int n = na * per;
  const int qb = (n + gridDim.x - 1) / gridDim.x;  // items per workgroup
  const int g0 = blockIdx.x * qb;
  if (g0 >= n) return;  // the whole workgroup, before its barrier
  const int g1 = min(n, g0 + qb);
  __shared__ int l_next;  // next item of the workgroup's run not yet taken
  // Everything that steers the loop is wave-uniform; readfirstlane keeps it in
  // scalar registers (values read from LDS would otherwise count as per-lane
  // and turn the loop into exec-masked control flow).
  const int lane = tid & 63, r = lane & 15, q = lane >> 4;
  const bool upper = r >= 8;  // which of the two whole-line loads holds this lane's first half
  // The next item of the workgroup's run (g1 once none is left); one lane
  // takes it from the counter.
  auto take = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&l_next, 1);
    const int nx = __builtin_amdgcn_readfirstlane(v);
    return nx < g1 ? nx : g1;
  };
  // Wave w starts on item g0 + w (its weight loads go out before the
  // activations are staged); the counter hands out the rest.
  const int first0 = g0 + __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool valid = first0 < g1;
  const int first = valid ? first0 : g1;
  const int nchunk = H / kChunkElems;  // H is a multiple of 1024
  const size_t wrb = H / 2, srb = H / 32;
  const size_t rows_per_expert = 2 * (size_t)I;

  // Number of 16-token passes of item `it`.
  auto passes_of = [&](int it) {
    const int a = it / per;
    const int nt = __builtin_amdgcn_readfirstlane(l_off[a + 1] - l_off[a]);
    return (nt + 15) >> 4;
  };

  // Prefetch cursor: item, pass, chunk, and this lane's two row pointers.
  int p_it = first, p_pass = 0, p_c = 0, p_npass = 0;
  if (valid) {
    const int a = first / per;
    p_npass = (__builtin_amdgcn_readfirstlane(row_off[a + 1] - row_off[a]) + 15) >> 4;
  }
  const uint8_t* pa[kNG];  // this lane's whole-line load A / B of chunk 0, per group
  const uint8_t* pb[kNG];
  const uint8_t* ps[kNG];
  auto p_rows = [&](int it, bool glob) {
    const int a = it / per, i0 = (it - a * per) * 16;
    const size_t row = (uint32_t)__builtin_amdgcn_readfirstlane(glob ? active_rows[a] : l_rows[a]);
    const uint8_t* wexp = w13 + row * rows_per_expert * wrb;
    const uint8_t* sexp = s13 + row * rows_per_expert * srb;
    pa[0] = wexp + (size_t)i0 * wrb + line_load_a(r, q, wrb);
    pb[0] = wexp + (size_t)i0 * wrb + line_load_b(r, q, wrb);
    ps[0] = sexp + (size_t)(i0 + r) * srb;
    pa[1] = wexp + (size_t)(I + i0) * wrb + line_load_a(r, q, wrb);
    pb[1] = wexp + (size_t)(I + i0) * wrb + line_load_b(r, q, wrb);
    ps[1] = sexp + (size_t)(I + i0 + r) * srb;
  };
  p_rows(valid ? first : g0, true);
  auto p_advance = [&]() {
    if (++p_c < nchunk) return;
    if (p_pass + 1 < p_npass) {  // next 16 tokens of the same item: its weights again
      p_c = 0;
      ++p_pass;
    } else {
      const int nx = take();
      if (nx < g1) {
        p_c = 0;
        p_pass = 0;
        p_it = nx;
        p_rows(nx, false);
        p_npass = passes_of(nx);
      } else {
        // Past the wavefront's last chunk the loads only keep the stream
        // unconditional: every wavefront cycles through the same quad of the
        // bank's first rows, which stays in the L2 (p_it unchanged tells the
        // consumer to stop). Its own last quad, just streamed past the L2,
        // was fetched again: ~24 MB per decode launch.
        p_c = nchunk - 4;
#pragma unroll
        for (int g = 0; g < kNG; ++g) {
          pa[g] = w13 + line_load_a(r, q, wrb);
          pb[g] = w13 + line_load_b(r, q, wrb);
        }
      }
    }
  };

  // Weight chunks run P ahead in a ring of P + 1 = 4 (only lo/hi of AChunk are
  // used). Scale bytes come in quads of chunks: at the start of every 4
  // chunks each lane takes the 8 scale bytes of one of the 4 chunks of its
  // row from the row's line (quad_from_line), and scale_quad turns them into
  // this lane's own pairs.
  static_assert(P == 3, "the ring cycle must match the 4-chunk scale quad");
  AChunk ring[P + 1][kNG];
  uint2 sraw[kNG];
  // A row's scale bytes are H/32 bytes: one 32-byte piece per quad, four
  // pieces per 128-byte line. The scale lines of the consumer's item (cur)
  // and of the line the prefetch cursor entered last (nxt); the consumer's
  // next quad and whether it starts a new line (then cur takes nxt).
  const int nq = nchunk >> 2;  // quads per row
  // Lane quarter q's piece of line L of its row; past the row's last quad a
  // lane reads piece 0 of the line instead (in bounds; never used).
  auto sline_off = [&](int L) {
    return 128 * L + 32 * (4 * L + q < nq ? q : 0);
  };
  uint4 sb_cur[kNG][2], sb_nxt[kNG][2];
  int s_quad = 0;
  bool s_new = false;
#pragma unroll
  for (int g = 0; g < kNG; ++g) {
    sb_cur[g][0] = *reinterpret_cast<const uint4*>(ps[g] + sline_off(0));
    sb_cur[g][1] = *reinterpret_cast<const uint4*>(ps[g] + sline_off(0) + 16);
    sb_nxt[g][0] = sb_cur[g][0];
    sb_nxt[g][1] = sb_cur[g][1];
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int g = 0; g < kNG; ++g) load_w(ring[p][g], pa[g], pb[g], p_c);
    p_advance();
  }

  {
    // Every thread issues all of its staging loads before its first LDS
    // store, so the workgroup waits for about one round trip to memory
    // instead of one per loop step. Loads and stores are unconditional: a
    // thread past the end of a table copies the table's last entry again (the
    // same value its owner writes), so no load sits under a branch. Slot
    // entries past the split's count are copied too (the slot list has T*k
    // entries); nothing reads them. na >= 1 here (the run is not empty).
    constexpr int kB = 8;  // granules of x per thread per batch
    const int gpr = kpad / 8, ng = T * gpr;
    for (int i0 = 0; i0 <= na || i0 < picks; i0 += kThreads) {
      const int i = i0 + tid;
      const int ir = i < na ? i : na - 1, io = i <= na ? i : na, is = i < picks ? i : picks - 1;
      const int vr = active_rows[ir], vo = row_off[io], vs = slots[is];
      l_rows[ir] = vr;
      l_off[io] = vo;
      l_slot[is] = vs;
      l_tok[is] = vs / k;
    }
    for (int b0 = 0; b0 < ng; b0 += kB * kThreads) {
      uint4 v[kB];
      int dst[kB];
      uint32_t pad = 0;  // bit u: granule u is zero padding past H
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int gi = min(b0 + u * kThreads + tid, ng - 1);
        const int n = gi / gpr, g = gi - n * gpr;
        v[u] = *reinterpret_cast<const uint4*>(x + (size_t)n * H + (g * 8 < H ? g * 8 : 0));
        pad |= (g * 8 >= H ? 1u : 0u) << u;
        dst[u] = lds_elem(n, kpad, g * 8);
      }
#pragma unroll
      for (int u = 0; u < kB; ++u)
        *reinterpret_cast<uint4*>(xs + dst[u]) = (pad >> u) & 1u ? make_uint4(0, 0, 0, 0) : v[u];
    }
    if (tid == 0) l_next = g0 + kThreads / 64;  // waves start on items g0 + wave
  }
  __syncthreads();


  if (!valid) return;  // no item for this wave (after the barrier)

  // The items the cursor took (and their 16-token passes) in order; nchunk is
  // a multiple of 4, so every pass starts at ring slot 0 and quad boundary,
  // and the prefetch cursor, P chunks ahead, crosses into the next pass or
  // item without a pause.
  for (int it = first;;) {
    const int a = it / per, i0 = (it - a * per) * 16;
    const int beg = __builtin_amdgcn_readfirstlane(l_off[a]);
    const int nt = __builtin_amdgcn_readfirstlane(l_off[a + 1]) - beg;
    for (int pass = 0; pass * 16 < nt; ++pass) {
      const int j = pass * 16 + r;
      const bool has = j < nt;
      const int xrow = l_tok[beg + (has ? j : 0)];
      f32x4 acc[kNG] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      for (int c = 0; c < nchunk; c += P + 1) {
        uint32_t sx[kNG], sy[kNG];
        if (s_new) {
#pragma unroll
          for (int g = 0; g < kNG; ++g) {
            sb_cur[g][0] = sb_nxt[g][0];
            sb_cur[g][1] = sb_nxt[g][1];
          }
        }
#pragma unroll
        for (int g = 0; g < kNG; ++g) sraw[g] = quad_from_line(sb_cur[g], r, q, s_quad & 3);
#pragma unroll
        for (int g = 0; g < kNG; ++g) scale_quad(sraw[g], sx[g], sy[g]);
#pragma unroll
        for (int u = 0; u <= P; ++u) {
          const int cc = c + u;
#pragma unroll
          for (int g = 0; g < kNG; ++g) load_w(ring[(u + P) % (P + 1)][g], pa[g], pb[g], p_c);
          p_advance();
          if (u == 0) {
            // the cursor now stands at the first chunk of the next quad
            s_quad = p_c >> 2;
            s_new = (p_c & 15) == 0;
            if (s_new) {  // a new item, pass or line: the rows' next scale line
              const int off = sline_off(p_c >> 4);
#pragma unroll
              for (int g = 0; g < kNG; ++g) {
                sb_nxt[g][0] = *reinterpret_cast<const uint4*>(ps[g] + off);
                sb_nxt[g][1] = *reinterpret_cast<const uint4*>(ps[g] + off + 16);
              }
            }
          }
          float sc[kNG][2];
#pragma unroll
          for (int g = 0; g < kNG; ++g) {
            const uint32_t pair = ((u & 1) ? sy[g] : sx[g]) >> ((u & 2) ? 16 : 0);
            sc[g][0] = e8m0_to_f32(pair & 0xffu);
            sc[g][1] = e8m0_to_f32((pair >> 8) & 0xffu);
          }
          const int e0 = cc * kChunkElems + 64 * q;
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const bf16x8 bv =
                *reinterpret_cast<const bf16x8*>(xs + lds_elem(xrow, kpad, e0 + 8 * m));
#pragma unroll
            for (int g = 0; g < kNG; ++g)
              acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  dequant8(own_word(ring[u][g], m, upper), sc[g][m >> 2]), bv, acc[g], 0, 0, 0);
          }
        }
      }
      // lane (r, q) holds i-rows i0 + 4q + v of the pass's token r
      if (has) {
        const size_t sl = l_slot[beg + j];
        uint32_t hb[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) hb[v] = f32_to_bf16_bits(silu_f32(acc[0][v]) * acc[1][v]);
        *reinterpret_cast<uint2*>(h_ws + sl * I + i0 + 4 * q) =
            make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
      }
    }
    if (p_it == it) break;  // the cursor took no further item
    it = p_it;
  }
}

template <int P>
hipError_t launch_p(const uint8_t* w13, const uint8_t* s13, int cap, const moe_split& sp,
                    const uint16_t* x, int T, int k, int H, int I, uint16_t* h_ws,
                    hipStream_t stream, int cus) {
  hipLaunchKernelGGL((ffn_gate_up_resident<P>), dim3(cus), dim3(kThreads),
                     resident_lds_bytes(T, k, H, cap), stream, w13, s13, sp.n_active,
                     sp.active_rows, sp.row_off, sp.slots, reinterpret_cast<const __bf16*>(x), T,
                     k, H, I, h_ws);
  return hipGetLastError();
}

}  // namespace

bool ffn_use_resident(int T, int k, int H, int cap, const void* s13) {
  // H a multiple of 1024: whole 4-chunk quads per row, 16-byte scale loads
  // inside the row; the scale tensor 16-byte aligned for those loads.
  return T >= 1 && T <= 16 && H % 1024 == 0 &&
         (reinterpret_cast<uintptr_t>(s13) & 15u) == 0 &&
         resident_lds_bytes(T, k, H, cap) <= kResidentMaxLds;
}

hipError_t launch_gate_up_resident(const uint8_t* w13, const uint8_t* s13, int cap, int on_host,
                                   const moe_split& sp, const uint16_t* x, int T, int k, int H,
                                   int I, uint16_t* h_ws, hipStream_t stream) {
  const int cus = device_cus();
  // A bank in host memory runs on kHostBankCUs workgroups (3 chunks in
  // flight per wavefront: enough to fill the host link); a device bank on the
  // other CUs.
  if (on_host) return launch_p<3>(w13, s13, cap, sp, x, T, k, H, I, h_ws, stream, kHostBankCUs);
  const int grid = cus > 2 * kHostBankCUs ? cus - kHostBankCUs : cus;
  return launch_p<3>(w13, s13, cap, sp, x, T, k, H, I, h_ws, stream, grid);
}

}  // namespace moe
