// moe_stream.hip — moe_forward with the routed experts streamed from host
// memory into a bounded cache of HBM expert slots, least recently used out
// first (colizig page, "Features": memory-tiered streaming with a bounded LRU
// expert cache, and the GPU backend's LRU VRAM weight cache; "What this
// project is trying to prove": most of a 512-expert model is cold at any
// instant, so experts stream across tiers instead of all being resident).
//
// Host side only: the kernels are moe_forward's, given a slot map (expert
// -> slot of the cache bank, -1 = not in this round). One call:
//   1. router, selection and permutation on the device (as moe_forward);
//   2. the group offsets come back to the host (the call waits for them):
//      they name the experts the call needs;
//   3. rounds: each takes up to `slots` of the still-unprocessed needed
//      experts, resident ones first; the missing ones are copied from the
//      caller's pinned host bank into the least recently used slots that no
//      expert of the round holds; the slot map goes up; the expert passes
//      run on the round's experts only (other groups exit at once). The
//      shared expert (resident, separate bank) runs in the first round;
//   4. the combine, once, over every expert's output.
// Copies and kernels share the caller's stream, so a slot is refilled only
// after the passes that read it. A call needing more experts than there are
// slots simply takes more rounds. The results are bit-identical to
// moe_forward's: the same kernels compute every group once.
#include <algorithm>
#include <vector>

#include "layer.hpp"

using namespace moe;

extern "C" moe_status moe_forward_streamed(const void* x, const float* router_w,
                                           const float* router_bias,
                                           const moe_expert_bank* host_experts,
                                           const moe_expert_bank* slot_bank,
                                           moe_expert_cache* cache, const moe_expert_bank* shared,
                                           int32_t top_k, void* out, const moe_config* cfg,
                                           void* workspace, size_t workspace_bytes_,
                                           void* stream) {
  Dims d;
  moe_status st = basic_dims(cfg, &d);
  if (st != MOE_OK) return st;
  if (top_k != cfg->top_k) return MOE_ERR_SHAPE;
  if (!x || !router_w || !out || !cache || !bank_ok(host_experts) || !bank_ok(slot_bank))
    return MOE_ERR_NULL;
  if (d.S && !bank_ok(shared)) return MOE_ERR_NULL;
  if (cache->slots < 1) return MOE_ERR_SHAPE;
  if (!cache->slot_expert || !cache->slot_used) return MOE_ERR_NULL;
  {  // the cache's contents must name distinct routed experts (or -1)
    std::vector<char> seen(d.E, 0);
    for (int i = 0; i < cache->slots; ++i) {
      const int e = cache->slot_expert[i];
      if (e == -1) continue;
      if (e < 0 || e >= d.E || seen[e]) return MOE_ERR_SHAPE;
      seen[e] = 1;
    }
  }
  st = expert_family_ok(d);
  if (st != MOE_OK) return st;
  if (d.T == 0) return MOE_OK;
  st = check_workspace(d, workspace, workspace_bytes_);
  if (st != MOE_OK) return st;

  const Work w = carve(d, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = enqueue_routing(d, x, router_w, router_bias, w, nullptr, s);
  if (st != MOE_OK) return st;

  // 2. which experts this call needs
  std::vector<int32_t> off(d.E + 2);
  if (hipMemcpyAsync(off.data(), w.offsets, off.size() * 4, hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MOE_ERR_HIP;
  std::vector<int> slot_of(d.E, -1);
  for (int i = 0; i < cache->slots; ++i)
    if (cache->slot_expert[i] >= 0) slot_of[cache->slot_expert[i]] = i;
  std::vector<int> pending;  // needed experts: resident ones first
  for (int pass = 0; pass < 2; ++pass)
    for (int e = 0; e < d.E; ++e)
      if (off[e + 1] > off[e] && (slot_of[e] >= 0) == (pass == 0)) pending.push_back(e);

  const size_t gu_w = (size_t)2 * d.I * d.H, dn_w = (size_t)d.H * d.I;
  const size_t gu_s = (size_t)(2 * d.I / d.B) * (d.H / d.B) * 4,
               dn_s = (size_t)(d.H / d.B) * (d.I / d.B) * 4;
  const moe_expert_bank* sh = d.S ? shared : nullptr;
  // one slot map per round, alive until the call's final synchronisation
  std::vector<std::vector<int32_t>> maps;
  size_t next = 0;
  int rounds = 0;
  do {
    // 3. this round's experts: up to `slots` pending ones (resident first)
    const size_t take = std::min(pending.size() - next, (size_t)cache->slots);
    std::vector<char> in_round(cache->slots, 0);
    std::vector<int> load;  // experts to copy in
    for (size_t i = next; i < next + take; ++i) {
      const int e = pending[i];
      if (slot_of[e] >= 0) in_round[slot_of[e]] = 1;
      else load.push_back(e);
    }
    // victims: slots no expert of this round holds, least recently used
    // (empty slots count as least recent)
    std::vector<int> victims;
    for (int i = 0; i < cache->slots; ++i)
      if (!in_round[i]) victims.push_back(i);
    std::stable_sort(victims.begin(), victims.end(), [&](int a, int b) {
      const int64_t ua = cache->slot_expert[a] < 0 ? -1 : cache->slot_used[a];
      const int64_t ub = cache->slot_expert[b] < 0 ? -1 : cache->slot_used[b];
      return ua < ub;
    });
    for (size_t j = 0; j < load.size(); ++j) {
      const int e = load[j], v = victims[j];
      if (cache->slot_expert[v] >= 0) slot_of[cache->slot_expert[v]] = -1;
      const moe_expert_bank& hb = *host_experts;
      const moe_expert_bank& sb = *slot_bank;
      if (hipMemcpyAsync(const_cast<uint8_t*>(sb.w_gate_up) + v * gu_w, hb.w_gate_up + e * gu_w,
                         gu_w, hipMemcpyHostToDevice, s) != hipSuccess ||
          hipMemcpyAsync(const_cast<uint8_t*>(sb.w_down) + v * dn_w, hb.w_down + e * dn_w, dn_w,
                         hipMemcpyHostToDevice, s) != hipSuccess ||
          hipMemcpyAsync(reinterpret_cast<uint8_t*>(const_cast<float*>(sb.s_gate_up)) + v * gu_s,
                         reinterpret_cast<const uint8_t*>(hb.s_gate_up) + e * gu_s, gu_s,
                         hipMemcpyHostToDevice, s) != hipSuccess ||
          hipMemcpyAsync(reinterpret_cast<uint8_t*>(const_cast<float*>(sb.s_down)) + v * dn_s,
                         reinterpret_cast<const uint8_t*>(hb.s_down) + e * dn_s, dn_s,
                         hipMemcpyHostToDevice, s) != hipSuccess)
        return MOE_ERR_HIP;
      cache->slot_expert[v] = e;
      slot_of[e] = v;
      cache->bytes_in += (int64_t)(gu_w + dn_w + gu_s + dn_s);
    }
    cache->misses += (int64_t)load.size();
    cache->hits += (int64_t)(take - load.size());
    maps.emplace_back(d.E + 1, -1);
    std::vector<int32_t>& map = maps.back();
    for (size_t i = next; i < next + take; ++i) {
      const int e = pending[i];
      map[e] = slot_of[e];
      cache->slot_used[slot_of[e]] = cache->calls;
    }
    map[d.E] = rounds == 0 ? 0 : -1;  // the shared group runs in the first round
    if (hipMemcpyAsync(w.slotmap, map.data(), map.size() * 4, hipMemcpyHostToDevice, s) !=
        hipSuccess)
      return MOE_ERR_HIP;
    const hipError_t e =
        d.mfma ? launch_experts_mfma(d, x, *slot_bank, sh, w, s, KernelEvents{}, w.slotmap)
               : launch_experts_gemv(d, x, *slot_bank, sh, w, s, KernelEvents{}, w.slotmap);
    if (e != hipSuccess) return MOE_ERR_HIP;
    next += take;
    ++rounds;
  } while (next < pending.size());

  // 4. one combine over every expert's output
  if (launch_combine(d, w, out, s) != hipSuccess) return MOE_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;  // the maps' lifetime
  cache->calls += 1;
  cache->rounds_last = rounds;
  return MOE_OK;
}
