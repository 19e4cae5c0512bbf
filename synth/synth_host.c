/*
 * Seeded synthetic inputs, host build. Test and benchmark infrastructure:
 * fills host buffers with the streams defined in synth_core.h. Large fills are
 * split over threads; each element depends only on (key, index), so the bytes
 * do not depend on the thread count.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -pthread
 */
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>

#include "synth_core.h"

typedef struct {
  void* out;
  int kind;
  uint64_t key, first, begin, end;
  float p0, p1;
  int32_t i0, i1;
} fill_job;

static void* fill_run(void* arg) {
  fill_job* j = (fill_job*)arg;
  for (uint64_t i = j->begin; i < j->end; ++i)
    syn_put(j->out, i, j->kind, j->key, j->first + i, j->p0, j->p1, j->i0, j->i1);
  return NULL;
}

uint64_t synth_key(uint64_t seed, uint32_t tag, uint32_t index) { return syn_key(seed, tag, index); }

uint64_t synth_draw(uint64_t key, uint64_t n) { return syn_draw(key, n); }

/* out[i] = element (first + i) of stream (key, kind), for i < count. */
int synth_fill(void* out, int kind, uint64_t key, uint64_t first, uint64_t count, float p0,
               float p1, int32_t i0, int32_t i1, int threads) {
  if (kind < SYN_F32_NORMAL || kind > SYN_E8M0) return -1;
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  if (count < (1u << 20)) threads = 1;
  fill_job jobs[64];
  pthread_t tids[64];
  uint64_t per = (count + (uint64_t)threads - 1) / (uint64_t)threads;
  int started = 0;
  for (int t = 0; t < threads; ++t) {
    uint64_t b = (uint64_t)t * per, e = b + per;
    if (b >= count) break;
    if (e > count) e = count;
    fill_job j = {out, kind, key, first, b, e, p0, p1, i0, i1};
    jobs[t] = j;
    if (t == threads - 1 || pthread_create(&tids[t], NULL, fill_run, &jobs[t]) != 0) {
      fill_run(&jobs[t]);
      tids[t] = 0;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (tids[t]) pthread_join(tids[t], NULL);
  return 0;
}
