"""MI355X-native Q4_0 fused-dequantization matmul and routed-expert MoE decode."""
