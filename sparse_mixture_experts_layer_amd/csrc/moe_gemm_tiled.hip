// Grouped expert GEMMs for large batches (prefill): LDS-staged tiles on bf16
// MFMA, the regime where each expert sees hundreds of rows.
//   gate/up:  h[r][f] = bf16(silu(x_r . Wg[f]) * (x_r . Wu[f]))   (r gathered via row_tok;
//             both dot products first bounded by the group's SwiGLU limit, if any)
//   down:     Y[r][n] = h_r . Wd[n]                                (fp32)
// h never leaves this pair of kernels, so it is stored in the order the down
// GEMM consumes it: 16-row x 32-feature fragments of 1 KiB in MFMA operand
// lane order, fragment (b, kb) at byte (b * hstride/32 + kb) * 1 KiB, where
// row-block b covers packed rows 16b .. 16b+15.  Group g's row r has packed
// row 16 * (ceil(offsets[g] / 16) + g) + r (each group starts on a fresh
// 16-row block; the gap before it is at most 16 rows).  The shared group's lo
// plane uses packed row r directly.  A wave's A load in the down GEMM is then
// one contiguous 1 KiB instead of 64-byte pieces of 16 rows, which measured
// 10-20% faster on these tiles.
// Expert FFN shape: llm-atlas "Step-3.5-Flash", "Champs bruts du config.json"
// (moe_intermediate_size, share_expert_dim, hidden_size); SiLU gating is the
// reading taken for the swiglu fields.
//
// Tile = TM rows x 256 weight rows, TM = 128 (4 waves, two workgroups per CU)
// or 256 (8 waves, one workgroup per CU; for experts with a few hundred rows:
// the CUs then pull a third fewer bytes per flop, which is what bounds these
// GEMMs).  Wave (wm, wn) owns rows 64*wm .. +63 and weight rows 128*wn .. +127
// (4 x 8 fragments of 16x16, 128 fp32 accumulators per lane).  K advances 32
// per stage through a 3-stage LDS ring: each stage is TM/16 A fragments (token
// rows, gathered straight from x by per-lane addresses) and 16 B fragments
// (packed weights), each 1 KiB and each written by one wave-wide global->LDS
// load in MFMA operand order, so every LDS read is a contiguous 1 KiB
// ds_read_b128 with no bank conflicts and no register staging.  Two stages are
// in flight while the third is multiplied, and the fragments of the next
// stage are read into registers during the current MFMAs.  Every SIMD runs two
// waves (of two workgroups, or of one 8-wave workgroup), so one's LDS traffic
// and barrier waits overlap the other's MFMAs.
//
// Precision: routed rows keep h in bf16 (one rounding, what the MFMA takes).
// The shared expert enters the output unweighted, so its rounding error would
// be the largest term of the output error: its h is stored as bf16 hi + lo
// (a second plane) and its down GEMM runs a second pass over lo.
//
// Tile order (which workgroups run together, hence what the L2s and the
// last-level cache share) differs between the two GEMMs; see the kernel.
#include "moe_common.hpp"
#include "moe_kernels.hpp"
#include "moe_lds.hpp"

namespace moe {
namespace {

constexpr int kTN = 256;                      // weight rows per tile
constexpr int kBFrags = kTN / 16;             // 16
constexpr int kXcds = 8;

// Per tile height TM: waves, fragments per stage, loads per wave and stage.
// NS: LDS ring stages (k-steps of loads in flight).
template <int TM, int NS>
struct TileShape {
  static constexpr int kWaves = TM / 32;                          // 4 or 8
  static constexpr int kAFrags = TM / 16;                         // 8 or 16
  static constexpr int kStageBytes = (kAFrags + kBFrags) * kFragBytes;
  static constexpr int kAL = kAFrags / kWaves;                    // 2
  static constexpr int kBL = kBFrags / kWaves;                    // 4 or 2
  static constexpr int kLoads = kAL + kBL;                        // 6 or 4
  // Y staging in the epilogue: MP fragment rows (16 rows each) per pass
  static constexpr int kMP = TM == 128 ? 2 : 1;
  static constexpr int kPitch = 128 * 4 + 16;                     // bytes per staged row
  static_assert(kWaves * kMP * 16 * kPitch <= NS * kStageBytes, "Y staging fits the ring");
  static_assert(kWaves * 16 * kFragBytes <= NS * kStageBytes, "h staging fits the ring");
};

template <int MODE, int TM>
__global__ __launch_bounds__(TM * 2, TM == 128 ? 2 : 1) void tiled_kernel(GemmGeom g, const uint16_t* __restrict__ a_src,
                                                    const int32_t* __restrict__ row_tok,
                                                    void* __restrict__ out, int hstride,
                                                    uint16_t* __restrict__ h_lo, int nblk) {
  // ring stages: 4 with 256-row tiles (down: 32 KiB stages, 128 KiB of ring;
  // gate/up: 4 B slots of 16 KiB and 3 A double slots of 32 KiB, all 160 KiB
  // of LDS), 3 with 128-row tiles
  constexpr int kStages = TM == 256 ? 4 : 3;
  using TS = TileShape<TM, kStages>;
  constexpr int kAFrags = TS::kAFrags, kStageBytes = TS::kStageBytes;
  constexpr int kAL = TS::kAL, kBL = TS::kBL, kLoadsPerStage = TS::kLoads;
  // Gate/up with 256-row tiles fetches the gathered x rows as whole 128-byte
  // lines: one wave-wide load takes 64 k of 8 rows (8 lanes per row) instead
  // of 32 k of 16 rows, which halves the cache lines each load touches.  A
  // line spans two k-steps, so A sits in kStages-1 double-step slots (TM rows
  // x 64 k each) beside a kStages-slot ring of B; the 16-byte chunks of a row are
  // XOR-swizzled by the row's index within its 8-row block so that the MFMA
  // operand reads stay free of bank conflicts.  Every other kernel keeps A
  // and B together per k-step.
  constexpr bool XL = MODE == 0 && TM == 256;
  constexpr int kBSlot = kBFrags * kFragBytes;                    // 16 KiB
  constexpr int kA2Bytes = TM * 128;                              // TM rows x 64 k
  constexpr int kA2Loads = kA2Bytes / kFragBytes / TS::kWaves;    // 4 per wave
  constexpr int kA2Slots = kStages - 1;
  constexpr int kLdsBytes = XL ? kStages * kBSlot + kA2Slots * kA2Bytes : kStages * kStageBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];

  // Work order.  Workgroups are dealt round-robin over the 8 XCDs (each with
  // its own L2; all share the last-level cache).  Inside an expert the
  // m-tiles are the fastest index (except for 128-row down tiles), so the
  // workgroups streaming one weight block start together.
  //   gate/up: the work list is cut into 8 contiguous chunks, one per XCD, so
  //     each XCD runs whole experts and its m-tiles share the weight blocks
  //     through L2 (the gathered x rows they also need stay in the
  //     last-level cache);
  //   down: round-robin in runs of two work items, so the 8 XCDs work on the
  //     same expert at once -- its weights are fetched from HBM once into the
  //     last-level cache and each XCD keeps a slice of them and the h tiles
  //     in its L2 -- while both m-tiles of one weight block (the two items of
  //     a run, for experts of up to two m-tiles) share that block through one
  //     L2 (1.5-2% faster than runs of one; whole chunks per XCD, as gate/up
  //     has them, measured 40% slower here).
  const int total = *g.ntiles * nblk;
  int w = (int)blockIdx.x;
  if (MODE == 1 && g.ksplit <= 1) {  // the grid is a multiple of 2 * kXcds
    const int slot = w / kXcds, x = w % kXcds;
    w = ((slot >> 1) * kXcds + x) * 2 + (slot & 1);
  }
  // a split K: the work list repeats once per part, part slowest (gate/up:
  // per part a grid slice of a multiple of 8 workgroups, dealt as below)
  const int nsplit = max(1, MODE == 1 ? g.ksplit : g.ksplit_gu);
  int split = 0;
  if (MODE == 1 && nsplit > 1) {
    split = w / total;
    if (split >= nsplit) return;
    w -= split * total;
  }
  if (MODE == 0) {
    int bid = (int)blockIdx.x;
    if (nsplit > 1) {
      const int per = (int)gridDim.x / nsplit;
      split = bid / per;
      bid -= split * per;
    }
    const int chunk = (total + kXcds - 1) / kXcds;
    const int slot = bid / kXcds;
    if (slot >= chunk) return;
    w = (bid % kXcds) * chunk + slot;
  }
  if (w >= total) return;
  const int v0 = g.tiles[w / nblk];
  const int group = tile_group(v0);
  if (MOE_DEBUG && (group < 0 || group > g.E)) {  // never written by the dispatch
    dbg_check(g.dbg, false, kDbgTile, v0);
    return;
  }
  int nb, mt;
  if (MODE == 0 || TM == 256) {  // m-tiles fastest inside the group, in blocks of kMB
    const int first = w / nblk - tile_m(v0);
    const int ntg = (g.counts[group] + TM - 1) / TM;
    const int local = w - first * nblk;
    // A group with many m-tiles (the shared expert, or a dense FFN as one
    // expert) walks them in blocks of kMB, all weight blocks per m block, so
    // that the workgroups running together cover a few m-tiles x a few weight
    // blocks rather than many m-tiles of one weight block (each k-step then
    // needs ~12 distinct operand slices instead of ~33 among 32 tiles);
    // groups of up to kMB m-tiles keep plain m-fastest order.
    constexpr int kMB = 8;
    const int full = ntg / kMB * kMB;
    if (local < full * nblk) {
      const int r = local % (kMB * nblk);
      nb = r / kMB;
      mt = local / (kMB * nblk) * kMB + r % kMB;
    } else {
      const int rem = ntg - full, r = local - full * nblk;
      nb = r / rem;
      mt = full + r % rem;
    }
  } else {                       // weight blocks fastest (measured better here)
    nb = w % nblk;
    mt = tile_m(v0);
  }
  const int row0 = g.offsets[group] + mt * TM;
  const int nrows = min(TM, g.counts[group] - mt * TM);
  // first packed h row-block of this tile (see the layout above)
  const int hb0 = (g.offsets[group] + 15) / 16 + group + mt * (TM / 16);
  const int hkb = hstride / 32;  // fragments per packed row-block
  if (nrows <= 0) return;
  const int width = group == g.E ? g.Is : g.I;
  const int H = g.H;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = MODE == 0 ? H : width;
  // k-steps of this workgroup: all of K, or part `split` of nsplit
  const int nk = K / 32 / nsplit;
  const int kbeg = split * nk;
  // weight blocks of 64 rows (gate/up: 32 features x {gate, up}; down: 64 outputs)
  const int nblocks = MODE == 0 ? width / 32 : H / 64;

  // this wave's two A fragments (rows 16*(2*wave) .. +31 of the tile); for the
  // shared group's down GEMM, pass 1 reads the lo plane
  static_assert(kAL == 2, "two A fragments per wave and stage");
  static_assert(!XL || kA2Loads == 4, "four A line loads per wave and double step");
  const bool shared = group == g.E;
  const float lim = shared ? g.limit_shared : g.limit;
  const int npass = (MODE == 1 && shared) ? 2 : 1;
  // routed rows of the down GEMM with y_bf16: lane l holds the gate weight and
  // the pair of the wave's row wm*64 + l, loaded now for the epilogue
  const bool yb = MODE == 1 && g.y_bf16 && !shared;
  float wrow = 0.f;
  int prow = 0;
  if (yb) {
    const int r = wm * 64 + lane;
    const int rc = row0 + (r < nrows ? r : 0);
    wrow = g.row_w[rc];
    prow = g.perm[rc];
  }
  size_t a_off[4];  // XL: one row per line load; otherwise the first two
  auto set_rows = [&](int pass) {
    if (XL) {
      // load u of this wave: tile rows 32*wave + 8u .. +7, lane -> row lane/8;
      // the lane fetches 16-byte chunk q of the row's 128 bytes and writes it
      // to LDS position lane, where the reader expects chunk (lane % 8) ^ (row % 8)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int r = 32 * wave + 8 * u + (lane >> 3);
        if (r >= nrows) r = 0;  // any valid row: its C row is never stored
        int tok = row_tok[row0 + r];
        dbg_check(g.dbg, tok >= 0 && tok < g.T, kDbgToken, tok);
        tok = tok < 0 ? 0 : (tok >= g.T ? g.T - 1 : tok);
        const int q = (lane & 7) ^ (lane >> 3);
        a_off[u] = (size_t)tok * H + (size_t)kbeg * 32 + q * 8;
      }
      return;
    }
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (MODE == 0) {
        int r = (2 * wave + f) * 16 + (lane & 15);
        if (r >= nrows) r = 0;  // any valid row: its C row is never stored
        int tok = row_tok[row0 + r];
        dbg_check(g.dbg, tok >= 0 && tok < g.T, kDbgToken, tok);
        tok = tok < 0 ? 0 : (tok >= g.T ? g.T - 1 : tok);
        a_off[f] = (size_t)tok * H + (size_t)kbeg * 32 + (lane >> 4) * 8;
      } else {
        // packed h: rows past nrows read the padding behind the group (inside
        // the buffer, whatever it holds); their C rows are never stored
        const int b = (pass == 0 ? hb0 : mt * (TM / 16)) + 2 * wave + f;
        a_off[f] = ((size_t)b * hkb + kbeg) * (kFragBytes / 2) + lane * 8;
      }
    }
  };
  // this wave's kBL B fragments: fragments kBL*wave .. of the tile's 16, i.e.
  // fragments (kBL*wave) % 4 .. of 64-row weight block nb*4 + kBL*wave/4
  // (each block is 4 KiB per k-step, its fragments contiguous).  A wave past
  // the last block loads block 0 instead (its columns are never stored), so
  // every wave issues the same number of loads per stage.
  const int bblk = nb * 4 + kBL * wave / 4;
  const uint8_t* bsrc = g.packed + (size_t)group * g.expert_bytes +
                        (MODE == 0 ? 0 : (size_t)2 * width * H * 2) +
                        (size_t)(bblk < nblocks ? bblk : 0) * (K / 32) * 4 * kFragBytes +
                        (size_t)kbeg * 4 * kFragBytes + (kBL * wave % 4) * kFragBytes +
                        lane * 16;

  const uint16_t* a_base = a_src;
  // elements from one k-step to the next: 32 along an x row, one fragment in packed h
  constexpr int kAStep = MODE == 0 ? 32 : kFragBytes / 2;
  // One LDS base per operand and stage; the fragments are told apart by the
  // instruction's immediate offset, which the global->LDS load adds to both
  // the global and the LDS address (two M0 writes per stage instead of six).
  auto issue_kstep = [&](int kk, int stage) {
    uint8_t* st = lds + stage * kStageBytes;
    uint8_t* la = st + 2 * wave * kFragBytes;
    load_frag<0>(a_base + a_off[0] + (size_t)kk * kAStep, la);
    load_frag<kFragBytes>(
        reinterpret_cast<const uint8_t*>(a_base + a_off[1] + (size_t)kk * kAStep) - kFragBytes, la);
    uint8_t* lb = st + (kAFrags + kBL * wave) * kFragBytes;
    const uint8_t* gb = bsrc + (size_t)kk * 4 * kFragBytes;
    load_frag<0>(gb, lb);
    load_frag<kFragBytes>(gb, lb);
    if (kBL == 4) {
      load_frag<2 * kFragBytes>(gb, lb);
      load_frag<3 * kFragBytes>(gb, lb);
    }
  };
  // XL: B of k-step kk in ring slot kk % kStages; A of k-steps 2d, 2d+1 in
  // double slot d % kA2Slots, issued with B of k-step 2d, kStages steps ahead
  // (that slot's previous double step, d - kA2Slots, was last read in step
  // 2d - kStages - 1, which every wave has left at the barrier of step
  // 2d - kStages that issues it)
  auto issue_b = [&](int kk, int slot) {
    uint8_t* lb = lds + slot * kBSlot + kBL * wave * kFragBytes;
    const uint8_t* gb = bsrc + (size_t)kk * 4 * kFragBytes;
    load_frag<0>(gb, lb);
    load_frag<kFragBytes>(gb, lb);
    if (kBL == 4) {
      load_frag<2 * kFragBytes>(gb, lb);
      load_frag<3 * kFragBytes>(gb, lb);
    }
  };
  auto issue_a2 = [&](int d, int dslot) {
    uint8_t* la = lds + kStages * kBSlot + dslot * kA2Bytes + 4 * wave * kFragBytes;
    const uint16_t* s0 = a_base + (size_t)d * 64;
    load_frag<0>(s0 + a_off[0], la);
    load_frag<kFragBytes>(reinterpret_cast<const uint8_t*>(s0 + a_off[1]) - kFragBytes, la);
    load_frag<2 * kFragBytes>(reinterpret_cast<const uint8_t*>(s0 + a_off[2]) - 2 * kFragBytes, la);
    load_frag<3 * kFragBytes>(reinterpret_cast<const uint8_t*>(s0 + a_off[3]) - 3 * kFragBytes, la);
  };
  // all loads of k-step kk, in the order the wait counts assume
  auto issue = [&](int kk) {
    if constexpr (XL) {
      issue_b(kk, kk % kStages);
      if ((kk & 1) == 0) issue_a2(kk >> 1, (kk >> 1) % kA2Slots);
    } else {
      issue_kstep(kk, kk % kStages);
    }
  };
  // XL: this lane's A operand (fragment row r = lane % 16, chunk c = lane / 16)
  // in a double slot: 8-row block r / 8, row r % 8, chunk c ^ (r % 8) (a
  // swizzle measured free of bank conflicts for these 16-byte reads; one that
  // also mixed in r / 8 was not); the odd k-step's chunks are 4 further
  // (bit 6 of the offset)
  const int xr = lane & 15;
  const int xa = (xr >> 3) * kFragBytes + (xr & 7) * 128 + 16 * ((lane >> 4) ^ (xr & 7));
  auto rd_a = [&](int kk, int m) {
    const uint8_t* p =
        XL ? lds + kStages * kBSlot + ((kk >> 1) % kA2Slots) * kA2Bytes + (wm * 4 + m) * 2 * kFragBytes +
                 (xa ^ ((kk & 1) * 64))
           : lds + (kk % kStages) * kStageBytes + (wm * 4 + m) * kFragBytes + lane * 16;
    return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
  };
  auto rd_b = [&](int kk, int j) {
    const uint8_t* p = XL ? lds + (kk % kStages) * kBSlot + (wn * 8 + j) * kFragBytes + lane * 16
                          : lds + (kk % kStages) * kStageBytes + (kAFrags + wn * 8 + j) * kFragBytes +
                                lane * 16;
    return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
  };
  // loads issued for k-step s (per wave)
  auto loads_of = [&](int s) { return XL ? kBL + ((s & 1) ? 0 : kA2Loads) : kLoadsPerStage; };

  f32x4 acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Pipeline, per k-step kk: wait until stage kk+1 has landed (own loads:
  // vmcnt; everyone's: barrier), refill the ring slot of stage kk (already in
  // registers) with stage kk+kStages, then run the MFMAs of stage kk while
  // reading stage kk+1 from LDS into registers: each B fragment is re-read in
  // place once its 4 MFMAs are issued, the A fragments go to a second register
  // set.  Global loads of kStages-1 stages stay in flight.
  bf16x8 a0[4], a1[4], b[8];
  auto step = [&](int kk, bf16x8(&ca)[4], bf16x8(&na)[4], bool do_issue, bool do_read, int vm) {
    wait_vm_lgkm0(vm);
    barrier();
    if (do_issue) issue(kk + kStages);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m][j] = mfma16(ca[m], b[j], acc[m][j]);
      if (do_read) {
        b[j] = rd_b(kk + 1, j);
        if (j < 4) na[j] = rd_a(kk + 1, j);
      }
    }
  };
  // loads issued after k-step kk+1's that may still be in flight at step kk:
  // those of k-steps kk+2 .. kk+kStages-1 that exist
  auto vm_at = [&](int kk) {
    int n = 0;
#pragma unroll
    for (int s = 2; s < kStages; ++s) n += kk + s < nk ? loads_of(kk + s) : 0;
    return n;
  };
  // the same in the main loop, for an even kk and for kk + 1 (XL: an even
  // k-step also carries a double step of A)
  auto vm_main = [](int parity) {
    int n = 0;
    for (int s = 2; s < kStages; ++s)
      n += XL ? kBL + (((parity + s) & 1) == 0 ? kA2Loads : 0) : kLoadsPerStage;
    return n;
  };
  constexpr int kVmEven = vm_main(0);
  constexpr int kVmOdd = vm_main(1);

  for (int pass = 0; pass < npass; ++pass) {
    // pass 1 (shared group, down GEMM) starts after the last step's barrier
    // of pass 0: every wave is done with the ring.
    set_rows(pass);
    a_base = pass == 0 ? a_src : h_lo;
    const int pro = nk < kStages ? nk : kStages;
    int vm0 = 0;
    for (int s = 0; s < pro; ++s) {
      issue(s);
      if (s > 0) vm0 += loads_of(s);
    }
    wait_vm_lgkm0(vm0);
    barrier();
#pragma unroll
    for (int m = 0; m < 4; ++m) a0[m] = rd_a(0, m);
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = rd_b(0, j);
    int kk = 0;
    for (; kk + kStages + 1 < nk; kk += 2) {
      step(kk, a0, a1, true, true, kVmEven);
      step(kk + 1, a1, a0, true, true, kVmOdd);
    }
    for (; kk < nk; kk += 2) {
      step(kk, a0, a1, kk + kStages < nk, kk + 1 < nk, vm_at(kk));
      if (kk + 1 < nk) step(kk + 1, a1, a0, kk + 1 + kStages < nk, kk + 2 < nk, vm_at(kk + 1));
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+i of each 16-row fragment, column lane%16
  if (MODE == 1) {
    // Y goes through LDS so that each lane stores 16 contiguous bytes and a
    // wave writes whole row segments (direct stores from the MFMA layout would
    // write 64-byte pieces, 4 bytes per lane).  The ring is idle: every wave
    // passed the last k-step's barrier after its last LDS read.  Each wave
    // stages its 64 x 128 block kMP fragment rows (16 rows each) at a time in
    // a private region; rows are padded by 16 bytes against bank conflicts.
    constexpr int kMP = TS::kMP, kPitch = TS::kPitch;
    uint8_t* stg = lds + wave * (kMP * 16 * kPitch);
    const int blk0 = nb * 4 + wn * 2;
    if (yb) {
      // routed rows of bf16 Y: weighted by their gate weight and rounded in
      // the MFMA layout (one shuffle per row for the weight), staged as bf16
      // (rows of 128 values, padded by 16 bytes), then stored 16 bytes (8
      // values) per lane at their pair's row
      constexpr int kPB = 128 * 2 + 16;
#pragma unroll
      for (int pass = 0; pass < 4 / kMP; ++pass) {
#pragma unroll
        for (int mm = 0; mm < kMP; ++mm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int lr = mm * 16 + (lane >> 4) * 4 + i;
            const float wr = __shfl(wrow, pass * kMP * 16 + lr);
#pragma unroll
            for (int j = 0; j < 8; ++j)
              *reinterpret_cast<uint16_t*>(stg + lr * kPB + (j * 16 + (lane & 15)) * 2) =
                  f32_to_bf16_bits(wr * acc[kMP * pass + mm][j][i]);
          }
        // kMP*16 rows x 16 chunks of 16 bytes, 64 chunks per wave-wide step
#pragma unroll
        for (int q = 0; q < kMP * 4; ++q) {
          const int idx = q * kWave + lane, lr = idx >> 4, ch = idx & 15;
          const int r = wm * 64 + pass * kMP * 16 + lr;
          const int blk = blk0 + (ch >> 3);
          const int pr = __shfl(prow, r - wm * 64);
          const u32x4 v = *reinterpret_cast<const u32x4*>(stg + lr * kPB + ch * 16);
          if (r < nrows && blk < nblocks)  // ordinary stores: 0.8% ahead of nontemporal ones
            *reinterpret_cast<u32x4*>(g.yb + (size_t)pr * H + (size_t)blk * 64 + (ch & 7) * 8) = v;
        }
      }
      return;
    }
    // fp32 rows: the shared group's (by token) or every row's (K-split planes,
    // fp32 activations)
#pragma unroll
    for (int pass = 0; pass < 4 / kMP; ++pass) {
#pragma unroll
      for (int mm = 0; mm < kMP; ++mm)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int lr = mm * 16 + (lane >> 4) * 4 + i, lc = j * 16 + (lane & 15);
            *reinterpret_cast<float*>(stg + lr * kPitch + lc * 4) = acc[kMP * pass + mm][j][i];
          }
      // kMP*16 rows x 32 chunks of 16 bytes, 64 chunks per wave-wide step
#pragma unroll
      for (int q = 0; q < kMP * 8; ++q) {
        const int idx = q * kWave + lane, lr = idx >> 5, ch = idx & 31;
        const f32x4 val = *reinterpret_cast<const f32x4*>(stg + lr * kPitch + ch * 16);
        const int r = wm * 64 + pass * kMP * 16 + lr;
        const int blk = blk0 + (ch >> 4);
        const size_t col = (size_t)blk * 64 + (ch & 15) * 4;
        if (r < nrows && blk < nblocks) {
          if (g.y_bf16)
            *reinterpret_cast<f32x4*>(g.ys + (size_t)(row0 + r - g.offsets[g.E]) * H + col) = val;
          else
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + split * g.y_plane +
                                      (size_t)(row0 + r) * H + col) = val;
        }
      }
    }
    return;
  }
  if (MODE == 0 && nsplit > 1) {  // partial sums of part `split`: gate and up rows of fp32
    float* gp = g.gu_part + split * g.gu_plane;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + m * 16 + (lane >> 4) * 4 + i;
        if (r >= nrows) continue;
        float* pr = gp + (size_t)(row0 + r) * 2 * hstride;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const int blk = nb * 4 + wn * 2 + jb;
          if (blk >= nblocks) continue;
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const int feat = 32 * blk + 16 * f + (lane & 15);
            pr[feat] = acc[m][jb * 4 + f][i];
            pr[hstride + feat] = acc[m][jb * 4 + 2 + f][i];
          }
        }
      }
    return;
  }
  // packed h: row rr of row-block b, feature 32*blk + 16*f + c sits in
  // fragment (b, blk) at lane rr + 16 * (2f + c/8), element c%8.  The wave's
  // 4 x 2 fragments (and their remainders, for the shared group) are put
  // together in its own 16 KiB of the ring, idle since every wave passed the
  // last k-step's barrier after its last LDS read, then stored whole: one
  // 16-byte store per lane and fragment instead of 16 two-byte ones.  A
  // fragment's rows past the tile are the group's padding rows (never stored
  // by the down GEMM); fragments wholly past the tile are not stored.
  uint16_t* sh = reinterpret_cast<uint16_t*>(lds + wave * 16 * kFragBytes);
  uint16_t* sl = sh + 8 * (kFragBytes / 2);
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = (lane >> 4) * 4 + i;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int at = (m * 2 + jb) * (kFragBytes / 2) +
                         (rr + 16 * (2 * f + ((lane & 15) >> 3))) * 8 + (lane & 7);
          const float hv = swiglu(acc[m][jb * 4 + f][i], acc[m][jb * 4 + 2 + f][i], lim);
          const uint16_t hi = f32_to_bf16_bits(hv);
          sh[at] = hi;
          if (shared) sl[at] = f32_to_bf16_bits(hv - bf16_bits_to_f32(hi));
        }
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (wm * 64 + m * 16 >= nrows) continue;
    const size_t b = (size_t)hb0 + wm * 4 + m, b_lo = (size_t)mt * (TM / 16) + wm * 4 + m;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      const int blk = nb * 4 + wn * 2 + jb;
      if (blk >= nblocks) continue;
      const int at = (m * 2 + jb) * (kFragBytes / 2) + lane * 8;
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) +
                                (b * hkb + blk) * (kFragBytes / 2) + lane * 8) =
          *reinterpret_cast<const u32x4*>(sh + at);
      if (shared)
        *reinterpret_cast<u32x4*>(h_lo + (b_lo * hkb + blk) * (kFragBytes / 2) + lane * 8) =
            *reinterpret_cast<const u32x4*>(sl + at);
    }
  }
}

// One thread per permuted row and 8 features: gate and up summed over the
// K parts in order, SwiGLU, and the 8 bf16 results stored as one 16-byte
// fragment lane of packed h (row r of group e at packed row
// 16 * (ceil(offsets[e] / 16) + e) + (r - offsets[e]); the shared group's
// remainder plane by its row).
__global__ __launch_bounds__(256) void gateup_reduce_kernel(GemmGeom g, int rows,
                                                            uint16_t* __restrict__ h,
                                                            uint16_t* __restrict__ h_lo,
                                                            int hstride) {
  const int per_row = hstride / 8;
  const int idx = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const int row = idx / per_row, f8 = (idx % per_row) * 8;
  if (row >= rows) return;
  // the group holding this row: the last e with offsets[e] <= row (groups
  // 0..E, offsets ascending; empty groups share an offset with the next)
  int lo = 0, hi = g.E;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (g.offsets[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int grp = lo;
  const bool shared = grp == g.E;
  const int width = shared ? g.Is : g.I;
  if (f8 >= width) return;
  const float lim = shared ? g.limit_shared : g.limit;
  f32x4 gs[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, us[2] = {gs[0], gs[1]};
  for (int sp = 0; sp < g.ksplit_gu; ++sp) {
    const float* pr = g.gu_part + sp * g.gu_plane + (size_t)row * 2 * hstride + f8;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      gs[q] += *reinterpret_cast<const f32x4*>(pr + 4 * q);
      us[q] += *reinterpret_cast<const f32x4*>(pr + hstride + 4 * q);
    }
  }
  uint16_t hb[8], lb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float hv = swiglu(gs[e / 4][e % 4], us[e / 4][e % 4], lim);
    hb[e] = f32_to_bf16_bits(hv);
    lb[e] = f32_to_bf16_bits(hv - bf16_bits_to_f32(hb[e]));
  }
  const int hkb = hstride / 32, kb = f8 / 32, lane_hi = 16 * ((f8 % 32) / 8);
  const int off = g.offsets[grp], rl = row - off;
  const size_t prow = (size_t)16 * ((off + 15) / 16 + grp) + rl;
  const size_t dst = ((prow / 16) * hkb + kb) * (kFragBytes / 2) + (prow % 16 + lane_hi) * 8;
  *reinterpret_cast<u32x4*>(h + dst) = u32x4{hb[0] | (uint32_t)hb[1] << 16, hb[2] | (uint32_t)hb[3] << 16,
                                             hb[4] | (uint32_t)hb[5] << 16, hb[6] | (uint32_t)hb[7] << 16};
  if (shared && h_lo) {
    const size_t dl = (((size_t)rl / 16) * hkb + kb) * (kFragBytes / 2) + (rl % 16 + lane_hi) * 8;
    *reinterpret_cast<u32x4*>(h_lo + dl) = u32x4{lb[0] | (uint32_t)lb[1] << 16, lb[2] | (uint32_t)lb[3] << 16,
                                                 lb[4] | (uint32_t)lb[5] << 16, lb[6] | (uint32_t)lb[7] << 16};
  }
}

}  // namespace

hipError_t launch_gateup_reduce(const GemmGeom& g, int rows, uint16_t* h, uint16_t* h_lo,
                                int hstride, hipStream_t s) {
  if (g.ksplit_gu < 2 || hstride % 32) return hipErrorInvalidValue;
  const long threads = (long)rows * (hstride / 8);
  dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  hipLaunchKernelGGL(gateup_reduce_kernel, grid, block, 0, s, g, rows, h, h_lo, hstride);
  return hipGetLastError();
}

hipError_t launch_gateup_tiled(const GemmGeom& g, const uint16_t* x, const int32_t* row_tok,
                               uint16_t* h, uint16_t* h_lo, int hstride, hipStream_t s) {
  const int tm = 16 * g.tg;
  if (tm != 128 && tm != 256) return hipErrorInvalidValue;
  const int wmax = g.I > g.Is ? g.I : g.Is;
  const int nblk = (2 * wmax + kTN - 1) / kTN;
  const int ns = g.ksplit_gu < 1 ? 1 : g.ksplit_gu;
  if ((g.H / 32) % (2 * ns) || (ns > 1 && !g.gu_part)) return hipErrorInvalidValue;
  const size_t items = (size_t)g.max_tiles * nblk;
  dim3 grid((unsigned)((items + kXcds - 1) / kXcds * kXcds * ns)), block(2 * tm);
  if (tm == 256)
    hipLaunchKernelGGL((tiled_kernel<0, 256>), grid, block, 0, s, g, x, row_tok, h, hstride, h_lo,
                       nblk);
  else
    hipLaunchKernelGGL((tiled_kernel<0, 128>), grid, block, 0, s, g, x, row_tok, h, hstride, h_lo,
                       nblk);
  return hipGetLastError();
}

hipError_t launch_down_tiled(const GemmGeom& g, const uint16_t* h, const uint16_t* h_lo,
                             int hstride, float* y, hipStream_t s) {
  const int tm = 16 * g.tg;
  if (tm != 128 && tm != 256) return hipErrorInvalidValue;
  const int nblk = (g.H + kTN - 1) / kTN;
  if (g.ksplit < 1 || (g.I / 32) % g.ksplit || (g.Is / 32) % g.ksplit) return hipErrorInvalidValue;
  const size_t items = (size_t)g.max_tiles * nblk * g.ksplit;
  const size_t q = 2 * kXcds;  // the runs of two of the work order need whole runs
  dim3 grid((unsigned)((items + q - 1) / q * q)), block(2 * tm);
  if (tm == 256)
    hipLaunchKernelGGL((tiled_kernel<1, 256>), grid, block, 0, s, g, h, nullptr, y, hstride,
                       const_cast<uint16_t*>(h_lo), nblk);
  else
    hipLaunchKernelGGL((tiled_kernel<1, 128>), grid, block, 0, s, g, h, nullptr, y, hstride,
                       const_cast<uint16_t*>(h_lo), nblk);
  return hipGetLastError();
}

}  // namespace moe
