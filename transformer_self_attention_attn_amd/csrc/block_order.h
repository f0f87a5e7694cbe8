// Order in which a forward kernel's query blocks are dealt to the chip.
// Internal; not installed.
//
// A launch has one workgroup per (batch, query head, query block of 128
// rows); the hardware deals workgroups to the 8 XCDs round-robin (block id
// mod 8) and, on each XCD, in increasing block id as slots free up.  Each
// XCD gets whole (batch, K/V head) groups, so a group's K/V tiles meet in
// one L2.  Under the causal mask a query block's work grows with its index:
// when the groups divide evenly over the XCDs, each XCD runs its blocks
// heaviest first across all of its groups (longest job first), so that no
// long diagonal block starts late; otherwise heaviest first within each
// group.  Where a group's K/V is large, the heaviest-first order goes band
// by band (qband query blocks each, enough blocks to fill the XCD's
// slots), one group at a time within a band, so that the XCD's L2 mostly
// holds one group's K/V.  The divisions by launch-fixed values go through
// fastdiv.h.
#pragma once

#include "fastdiv.h"

namespace miattn {

constexpr int kOrderXcds = 8;  // MI355X: 8 accelerator complex dies

struct BlockOrder {
  int total;   // blocks: B * Hkv * G * nqb
  int G;       // query heads per K/V head
  int nqb;     // query blocks per head
  int Hkv;     // K/V heads
  int qband;   // query blocks per band (longest-first order)
  int gpx;     // groups per XCD (longest-first order)
  int lpt;     // 1: longest first across each XCD's groups
  int causal;  // 1: heaviest (highest) query block first
  // divisors: blocks of a band across an XCD's groups (gpx qband G), of one
  // group's band (qband G), G, Hkv, blocks of one group (G nqb)
  UDiv dv_band, dv_bs, dv_g, dv_hkv, dv_grp;
};

// kv_group_bytes: K and V bytes of one (batch, K/V head) group;
// slots_per_xcd: workgroups one XCD runs at once.
inline BlockOrder make_block_order(int B, int Hkv, int G, int nqb,
                                   bool causal, long long kv_group_bytes,
                                   int slots_per_xcd) {
  BlockOrder o{};
  o.total = B * Hkv * G * nqb;
  o.G = G;
  o.nqb = nqb;
  o.Hkv = Hkv;
  o.causal = causal ? 1 : 0;
  const int ngrp = B * Hkv;
  o.lpt = (causal && ngrp % kOrderXcds == 0) ? 1 : 0;
  o.gpx = ngrp / kOrderXcds;
  o.qband = 1;
  if (o.lpt && kv_group_bytes >= (1LL << 20)) {
    for (int qb = 1; qb <= nqb; ++qb)
      if (nqb % qb == 0) {
        o.qband = qb;
        if (qb * G >= slots_per_xcd) break;
      }
  }
  o.dv_band = make_udiv(o.gpx * o.qband * G);
  o.dv_bs = make_udiv(o.qband * G);
  o.dv_g = make_udiv(G);
  o.dv_hkv = make_udiv(Hkv);
  o.dv_grp = make_udiv(G * nqb);
  return o;
}

struct BlockPos {
  int b, hk, hh, qb;  // batch, K/V head, head within the group, query block
};

MIATTN_FD_HD inline BlockPos block_pos(int bid, const BlockOrder& o) {
  const int xcd = (int)((unsigned)bid % kOrderXcds);
  const int slot = (int)((unsigned)bid / kOrderXcds);
  int grp, qrank, hh;
  if (o.lpt) {
    const int bs = o.qband * o.G;  // blocks of one group in a band
    const int band = udiv(slot, o.dv_band);
    const int r1 = slot - band * o.gpx * bs;
    const int gi = udiv(r1, o.dv_bs);
    const int r2 = r1 - gi * bs;
    const int r2g = udiv(r2, o.dv_g);
    qrank = band * o.qband + r2g;
    grp = xcd * o.gpx + gi;
    hh = r2 - r2g * o.G;
  } else {
    const int per = (int)((unsigned)o.total / kOrderXcds);
    const int rem = (int)((unsigned)o.total % kOrderXcds);
    const int lid = xcd * per + (xcd < rem ? xcd : rem) + slot;
    grp = udiv(lid, o.dv_grp);
    const int r0 = lid - grp * o.G * o.nqb;
    qrank = udiv(r0, o.dv_g);
    hh = r0 - qrank * o.G;
  }
  BlockPos pos;
  pos.qb = o.causal ? (o.nqb - 1 - qrank) : qrank;
  pos.b = udiv(grp, o.dv_hkv);
  pos.hk = grp - pos.b * o.Hkv;
  pos.hh = hh;
  return pos;
}

}  // namespace miattn
