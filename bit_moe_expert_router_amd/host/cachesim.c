/* cachesim.c -- replay of expert-cache policies over routing traces (host tool).
 *
 * The pages size a GPU expert cache per layer and compare replacement policies by
 * misses per token on recorded routing traces (page "GLM-5.3-Flash EXL3 3.05bpw
 * on 1x RTX PRO 6000 - GPU expert cache, host-RAM streaming", field
 * config.expert_cache.policy_data: static, LRU, LFU with decay 0.995 and Belady at
 * 170 slots; page "0xSero/glm53-flash-offload", paragraph "Elastic CLOCK expert
 * cache": a CLOCK cache).  This file replays the same policies over any trace so
 * that a slot count and a policy can be chosen for the device-side cache.
 *
 * Trace: for step s (one decode step) and layer l, the distinct experts the step
 * needs in that layer: trace[off[s*L + l] .. off[s*L + l + 1]), ids in [0, E).
 * Every layer has its own cache of S slots.  At a step, each needed expert that
 * is resident is a hit; the others are misses, each admitted into a free slot or
 * in place of a victim that the step does not need (when every resident expert is
 * needed, the miss is served without admission).  Policies:
 *   MOE_SIM_STATIC: the S experts of the layer used in most steps of the whole
 *     trace (ties to the lower id) are resident from the start; nothing is
 *     admitted.
 *   MOE_SIM_LRU:    victim = least recently used.
 *   MOE_SIM_LFU:    every expert's score decays by `decay` per step and gains 1
 *     per step that uses it (scores kept for all experts, resident or not);
 *     victim = lowest score, ties to the least recently used, then the lower id.
 *   MOE_SIM_BELADY: victim = the resident expert whose next use is furthest away
 *     (never used again counts as infinitely far), ties to the lower id: the
 *     fewest misses any policy can reach on the trace.
 *   MOE_SIM_CLOCK:  slots in a ring with one reference bit each (set on a hit and
 *     on admission); the hand skips and clears set bits and takes the first slot
 *     whose bit is clear and whose expert the step does not need.
 * Outputs misses[s] (over all layers) for every step.  Returns total misses, or
 * -1 on bad arguments.  Plain C, no threads: a few million lookups per second. */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { MOE_SIM_STATIC = 0, MOE_SIM_LRU = 1, MOE_SIM_LFU = 2, MOE_SIM_BELADY = 3, MOE_SIM_CLOCK = 4 };

typedef struct {
  int32_t* slot_of;   /* [E]: slot holding the expert, -1 if not resident */
  int32_t* expert;    /* [S]: expert in the slot, -1 if free             */
  int64_t* last;      /* [E]: last step that used the expert             */
  double* score;      /* [E]: LFU score                                  */
  uint8_t* ref;       /* [S]: CLOCK reference bits                       */
  uint8_t* needed;    /* [E]: needed by the current step                 */
  int32_t hand;
} layer_state;


int64_t moe_cachesim(const int32_t* trace, const int32_t* off, int64_t steps, int32_t L,
                     int32_t E, int32_t S, int32_t policy, double decay, int64_t* misses) {
  if (!trace || !off || !misses || steps < 0 || L <= 0 || E <= 0 || S < 0 || policy < 0 ||
      policy > MOE_SIM_CLOCK)
    return -1;
  for (int64_t s = 0; s < steps; ++s) misses[s] = 0;
  int64_t total = 0;
  layer_state st;
  st.slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  st.expert = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
  st.last = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  st.score = (double*)malloc(sizeof(double) * (size_t)E);
  st.ref = (uint8_t*)malloc((size_t)(S > 0 ? S : 1));
  st.needed = (uint8_t*)malloc((size_t)E);
  int64_t* uses = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  /* Belady: the next step using the expert of each trace entry, and per expert
   * the next use after its latest one */
  const int64_t n_entries = off[steps * L];
  int64_t* nxt_entry = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_entries > 0 ? n_entries : 1));
  int64_t* nxt = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  for (int32_t l = 0; l < L; ++l) {
    for (int32_t e = 0; e < E; ++e) {
      st.slot_of[e] = -1;
      st.last[e] = -1;
      st.score[e] = 0.0;
      st.needed[e] = 0;
    }
    for (int32_t k = 0; k < S; ++k) {
      st.expert[k] = -1;
      st.ref[k] = 0;
    }
    st.hand = 0;
    if (policy == MOE_SIM_BELADY) {
      for (int32_t e = 0; e < E; ++e) uses[e] = INT64_MAX; /* next step seen, backwards */
      for (int64_t s = steps - 1; s >= 0; --s) {
        for (int32_t i = off[s * L + l]; i < off[s * L + l + 1]; ++i) nxt_entry[i] = uses[trace[i]];
        for (int32_t i = off[s * L + l]; i < off[s * L + l + 1]; ++i) uses[trace[i]] = s;
      }
    }
    if (policy == MOE_SIM_STATIC) {  /* the S experts used in most steps */
      for (int32_t e = 0; e < E; ++e) uses[e] = 0;
      for (int64_t s = 0; s < steps; ++s)
        for (int32_t i = off[s * L + l]; i < off[s * L + l + 1]; ++i) uses[trace[i]]++;
      for (int32_t k = 0; k < S && k < E; ++k) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e)
          if (st.slot_of[e] < 0 && (best < 0 || uses[e] > uses[best])) best = e;
        st.slot_of[best] = k;
        st.expert[k] = best;
      }
    }
    for (int64_t s = 0; s < steps; ++s) {
      const int32_t b = off[s * L + l], en = off[s * L + l + 1];
      if (policy == MOE_SIM_LFU)
        for (int32_t e = 0; e < E; ++e) st.score[e] *= decay;
      for (int32_t i = b; i < en; ++i) st.needed[trace[i]] = 1;
      for (int32_t i = b; i < en; ++i) {
        const int32_t e = trace[i];
        if (policy == MOE_SIM_LFU) st.score[e] += 1.0;
        if (policy == MOE_SIM_BELADY) nxt[e] = nxt_entry[i];
        if (st.slot_of[e] >= 0) {  /* hit */
          if (policy == MOE_SIM_CLOCK) st.ref[st.slot_of[e]] = 1;
          st.last[e] = s;
          continue;
        }
        misses[s]++;
        total++;
        st.last[e] = s;
        if (policy == MOE_SIM_STATIC || S == 0) continue;
        /* a free slot, else a victim the step does not need */
        int32_t k = -1;
        for (int32_t q = 0; q < S; ++q)
          if (st.expert[q] < 0) {
            k = q;
            break;
          }
        if (k < 0) {
          if (policy == MOE_SIM_CLOCK) {
            for (int32_t n = 0; n < 2 * S && k < 0; ++n) {
              const int32_t q = st.hand;
              st.hand = (st.hand + 1) % S;
              if (st.needed[st.expert[q]]) continue;
              if (st.ref[q]) {
                st.ref[q] = 0;
                continue;
              }
              k = q;
            }
          } else {
            int64_t best_key = 0;
            double best_score = 0.0;
            for (int32_t q = 0; q < S; ++q) {
              const int32_t v = st.expert[q];
              if (st.needed[v]) continue;
              int take = 0;
              if (k < 0) {
                take = 1;
              } else if (policy == MOE_SIM_LRU) {
                take = st.last[v] < best_key || (st.last[v] == best_key && v < st.expert[k]);
              } else if (policy == MOE_SIM_LFU) {
                take = st.score[v] < best_score ||
                       (st.score[v] == best_score &&
                        (st.last[v] < best_key || (st.last[v] == best_key && v < st.expert[k])));
              } else { /* Belady: furthest next use */
                take = nxt[v] > best_key || (nxt[v] == best_key && v < st.expert[k]);
              }
              if (take) {
                k = q;
                best_score = st.score[v];
                best_key = policy == MOE_SIM_BELADY ? nxt[v] : st.last[v];
              }
            }
          }
          if (k < 0) continue; /* every resident expert is needed: not admitted */
          st.slot_of[st.expert[k]] = -1;
        }
        st.slot_of[e] = k;
        st.expert[k] = e;
        st.ref[k] = 1;
      }
      for (int32_t i = b; i < en; ++i) st.needed[trace[i]] = 0;
    }
  }
  free(st.slot_of);
  free(st.expert);
  free(st.last);
  free(st.score);
  free(st.ref);
  free(st.needed);
  free(uses);
  free(nxt_entry);
  free(nxt);
  return total;
}
