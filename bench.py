"""placeholder: replaced below"""
def q8_weight_bytes(N, K):
    return N * K // 32 * 34
