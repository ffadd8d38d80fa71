// LDS bank model of gfx950 and the conflict simulation of one transpose tile.
//
// The swizzle chooser of the register-staged permute simulates the shared-memory bank pattern
// and keeps the smallest XOR bit count that leaves both the read and the write phase
// conflict-free (TVM TIRx docs, "permute_layout", Algorithm step 2).  That page models 32 banks
// of 4 bytes and a 32-lane warp.  gfx950's LDS was measured instead (a one-wave probe per access
// pattern, cycles per access and SQ_LDS_BANK_CONFLICT): reads and writes of 1, 2 and 4 bytes use
// 32 banks and serve 32 lanes at a time; 8-byte reads 64 banks x 32 lanes; 8-byte writes
// 32 banks x 16 lanes; 16-byte reads 64 banks x 16 lanes; 16-byte writes 32 banks x 8 lanes.
// Inside one such lane group a bank that must deliver n different dwords costs n - 1 extra
// cycles; lanes asking for the same dword share it.
#include <algorithm>
#include <vector>

#include "plan.hpp"

namespace tc {

BankGeom gfx950_bank_geom(bool write, int width) {
  if (width <= 4) return {32, 32};
  if (width == 8) return write ? BankGeom{32, 16} : BankGeom{64, 32};
  return write ? BankGeom{32, 8} : BankGeom{64, 16};
}

int64_t lds_conflict_cycles(const int64_t* byte_addr, const bool* active, int lanes, int width, bool write) {
  const BankGeom g = gfx950_bank_geom(write, width);
  int64_t total = 0;
  // Distinct dwords per bank within one lane group.  A lane's dwords are consecutive, so it adds
  // at most one dword to a bank: a bank holds at most `group` (<= 32) entries.
  int64_t seen[64][32];
  int cnt[64];
  for (int g0 = 0; g0 < lanes; g0 += g.group) {
    std::fill(cnt, cnt + g.banks, 0);
    int worst = 0;
    for (int l = g0; l < std::min(lanes, g0 + g.group); ++l) {
      if (active && !active[l]) continue;
      const int64_t first = byte_addr[l] / 4, last = (byte_addr[l] + width - 1) / 4;
      for (int64_t wd = first; wd <= last; ++wd) {
        const int bank = int(((wd % g.banks) + g.banks) % g.banks);
        int i = 0;
        while (i < cnt[bank] && seen[bank][i] != wd) ++i;
        if (i == cnt[bank]) {
          seen[bank][cnt[bank]++] = wd;
          worst = std::max(worst, cnt[bank]);
        }
      }
    }
    total += worst > 0 ? worst - 1 : 0;
  }
  return total;
}

bool finish_geom(TileGeom* g) {
  if (g->eb <= 0 || g->vb < g->eb || g->vb % g->eb) return false;
  if (g->U == 0) g->U = g->eb < 4 ? 4 : g->eb;
  if ((g->U != 4 && g->U != 8 && g->U != 16) || g->U < g->eb) return false;
  g->B = g->U / g->eb;
  g->VE = g->vb / g->eb;
  if (g->vb < g->U) return false;  // a store vector covers whole units
  for (int v : {g->TR, g->TC, g->NB})
    if (v <= 0 || (v & (v - 1))) return false;
  if (g->TR % g->VE || g->TC % g->VE || g->TR % g->B) return false;
  if (int64_t(g->TR) * g->TC * g->NB * g->eb != g->tile_bytes) return false;
  const int per_load = g->NT * g->vb * g->B, per_store = g->NT * g->vb;
  if (g->tile_bytes % per_load || g->tile_bytes % per_store) return false;
  g->loads = g->tile_bytes / per_load;
  g->stores = g->tile_bytes / per_store;
  g->ww = std::min(16, g->VE * g->U);
  g->rw = g->U;
  if (g->TRu() < g->RPV()) return false;
  const int chunks = g->TC / g->CW();
  if (g->k < 0 || g->tbit < 0 || g->shift < 0) return false;
  if (g->k > 0 && (1 << (g->k + g->tbit)) > chunks) return false;
  if (g->cmask < 0 || (g->cmask && (g->cshift < 1 || g->cmask >= (1 << g->cshift) || (1 << g->cshift) >= chunks)))
    return false;
  return true;
}

// Lane -> LDS address of both phases; must match the transpose kernel exactly.
// Load phase: access a = f*NT + t over the tile in source order (nb, ru, cv) with cv fastest;
// it writes the VE units of columns cv*VE.. of unit-row ru, in instructions of ww bytes.
// Store phase: access a = f*NT + t in destination order (nb, c, rv) with rv fastest; it reads
// the RPV units ru = rv*RPV + v of column c, one rw-byte instruction each.
void simulate_tile(const TileGeom& g, int64_t* write_cycles, int64_t* read_cycles, int64_t limit) {
  const int nCV = g.TC / g.VE;
  const int TRu = g.TRu();
  const int RPV = g.RPV();
  const int nRV = TRu / RPV;
  const int CW = g.CW();
  const int per_access_w = g.VE / CW;  // write instructions per load access
  int64_t addr[kWave];
  int64_t wc = 0, rc = 0;
  for (int w = 0; w < g.NT / kWave; ++w) {
    for (int f = 0; f < g.loads; ++f)
      for (int q = 0; q < per_access_w; ++q) {
        for (int l = 0; l < kWave; ++l) {
          const int a = f * g.NT + w * kWave + l;
          const int cv = a % nCV, ru = (a / nCV) % TRu, nb = a / (nCV * TRu);
          addr[l] = g.unit_addr(nb, ru, cv * g.VE + q * CW) * g.U;
        }
        wc += lds_conflict_cycles(addr, nullptr, kWave, g.ww, true);
        if (limit >= 0 && wc + rc >= limit) goto done;
      }
    for (int f = 0; f < g.stores; ++f)
      for (int v = 0; v < RPV; ++v) {
        for (int l = 0; l < kWave; ++l) {
          const int a = f * g.NT + w * kWave + l;
          const int rv = a % nRV, c = (a / nRV) % g.TC, nb = a / (nRV * g.TC);
          addr[l] = g.unit_addr(nb, rv * RPV + v, c) * g.U;
        }
        rc += lds_conflict_cycles(addr, nullptr, kWave, g.rw, false);
        if (limit >= 0 && wc + rc >= limit) goto done;
      }
  }
done:
  *write_cycles = wc;
  *read_cycles = rc;
}

bool tile_wave_local(const TileGeom& g) {
  // owner wave of every LDS unit (by its unswizzled position: the swizzle is a bijection)
  const int nCV = g.TC / g.VE, TRu = g.TRu(), RPV = g.RPV(), nRV = TRu / RPV;
  std::vector<int> owner(size_t(g.NB) * TRu * g.TC, -1);
  for (int f = 0; f < g.loads; ++f)
    for (int t = 0; t < g.NT; ++t) {
      const int a = f * g.NT + t;
      const int cv = a % nCV, ru = (a / nCV) % TRu, nb = a / (nCV * TRu);
      for (int j = 0; j < g.VE; ++j) owner[(size_t(nb) * TRu + ru) * g.TC + cv * g.VE + j] = t / kWave;
    }
  for (int f = 0; f < g.stores; ++f)
    for (int t = 0; t < g.NT; ++t) {
      const int a = f * g.NT + t;
      const int rv = a % nRV, c = (a / nRV) % g.TC, nb = a / (nRV * g.TC);
      for (int v = 0; v < RPV; ++v)
        if (owner[(size_t(nb) * TRu + rv * RPV + v) * g.TC + c] != t / kWave) return false;
    }
  return true;
}

}  // namespace tc
