/* The host entry points of the C ABI called from plain C: nothing but the
 * public header and the shared library.  Every result is printed as one text
 * line, "<name> <values...>", for the test that builds and runs this program
 * to compare with the oracle.  Exit status 0 when every call returned what
 * the header promises, 1 otherwise (the failing call is named on stderr). */
#include <stdio.h>
#include <stdlib.h>

#include "ringattn.h"

static int failures = 0;

static void expect(int32_t status, int32_t want, const char* what) {
  if (status != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d: %s\n", what, (int)status,
            cp_status_string(status), (int)want, cp_last_error());
    ++failures;
  }
}

static void print_i64(const char* name, const int64_t* a, int64_t n) {
  printf("%s", name);
  for (int64_t i = 0; i < n; ++i) printf(" %lld", (long long)a[i]);
  printf("\n");
}

static void print_i32(const char* name, const int32_t* a, int64_t n) {
  printf("%s", name);
  for (int64_t i = 0; i < n; ++i) printf(" %d", (int)a[i]);
  printf("\n");
}

int main(void) {
  printf("abi %d\n", (int)cp_abi_version());

  /* cp_partition: two requests (10 and 7 tokens), cp 2, every rank; the
   * first call only asks for the lengths. */
  const int64_t lens[2] = {10, 7};
  for (int32_t rank = 0; rank < 2; ++rank) {
    int64_t local_len = 0, restore_len = 0;
    expect(cp_partition(lens, 2, 2, rank, NULL, &local_len, NULL, &restore_len), CP_OK, "cp_partition sizes");
    int64_t* local = malloc(sizeof(int64_t) * (size_t)(local_len > 0 ? local_len : 1));
    int64_t* restore = malloc(sizeof(int64_t) * (size_t)(restore_len > 0 ? restore_len : 1));
    if (!local || !restore) return 1;
    expect(cp_partition(lens, 2, 2, rank, local, &local_len, restore, &restore_len), CP_OK, "cp_partition");
    printf("partition_rank %d\n", (int)rank);
    print_i64("local", local, local_len);
    print_i64("restore", restore, restore_len);
    free(local);
    free(restore);
  }

  /* cp_slot_mapping: 40 positions, block 8, interleave 2, pcp 2, dcp 2,
   * identity table and then a table of 5 physical blocks. */
  int64_t pos[40];
  int32_t dev[40];
  int64_t slot[40];
  for (int i = 0; i < 40; ++i) pos[i] = 3 * i + 1;
  expect(cp_slot_mapping(pos, 40, 8, 2, 2, 2, NULL, 0, dev, slot), CP_OK, "cp_slot_mapping");
  print_i32("dev", dev, 40);
  print_i64("slot", slot, 40);
  const int32_t table[5] = {4, 0, 3, 1, 2};
  expect(cp_slot_mapping(pos, 40, 8, 2, 2, 2, table, 5, dev, slot), CP_OK, "cp_slot_mapping table");
  print_i32("dev_table", dev, 40);
  print_i64("slot_table", slot, 40);
  /* block_size not a multiple of the interleave: rejected */
  expect(cp_slot_mapping(pos, 40, 8, 3, 2, 2, NULL, 0, dev, slot), CP_EINVAL, "cp_slot_mapping bad interleave");

  /* cp_ring_schedule: rank 2 of 4 */
  int32_t src[4], parts[8];
  expect(cp_ring_schedule(2, 4, src, parts), CP_OK, "cp_ring_schedule");
  print_i32("ring_src", src, 4);
  print_i32("ring_parts", parts, 8);

  /* cp_classify: a FULL, a DIAG and a SKIP pair under the causal mask */
  int32_t cls[3];
  expect(cp_classify(100, 50, 0, 64, CP_MASK_CAUSAL, &cls[0]), CP_OK, "cp_classify full");
  expect(cp_classify(100, 50, 120, 10, CP_MASK_CAUSAL, &cls[1]), CP_OK, "cp_classify diag");
  expect(cp_classify(100, 50, 150, 10, CP_MASK_CAUSAL, &cls[2]), CP_OK, "cp_classify skip");
  print_i32("classify", cls, 3);

  /* cp_reorg_index: the two requests on 2 x 1 devices, block 4, interleave 2 */
  int64_t n_src = 0;
  expect(cp_reorg_index(lens, 2, 4, 2, 2, 1, NULL, &n_src, NULL, 0), CP_OK, "cp_reorg_index size");
  int64_t* rows = malloc(sizeof(int64_t) * (size_t)(n_src > 0 ? n_src : 1));
  int64_t dev_lens[4];
  if (!rows) return 1;
  expect(cp_reorg_index(lens, 2, 4, 2, 2, 1, rows, &n_src, dev_lens, 4), CP_OK, "cp_reorg_index");
  print_i64("reorg_src", rows, n_src);
  print_i64("reorg_dev_lens", dev_lens, 4);
  free(rows);

  printf("status_string %s\n", cp_status_string(CP_EINVAL));
  return failures == 0 ? 0 : 1;
}
